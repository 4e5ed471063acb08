"""The allocation-free split-K entry point (w24_gemm_f16_splitk_static),
called through the C ABI: its output equals w24_gemm_f16_splitk's (same
kernels, same split order: bit-identical) and meets the oracle's bounds, on
two calls in a row, the second with a smaller input (the static scratch keeps
the first call's partials, which the second must fully overwrite)."""

import ctypes as ct

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


def T(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def H(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _static_call(lib, A, vals, meta, C, splits):
    """The entry point through its raw C signature."""
    import torch
    M, K = A.shape
    N = vals.shape[0]
    return lib.load().w24_gemm_f16_splitk_static(
        ct.c_void_p(A.data_ptr()), ct.c_void_p(vals.data_ptr()), ct.c_void_p(meta.data_ptr()),
        ct.c_void_p(C.data_ptr()), M, N, K, splits, ct.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_scratch_matches_workspace_call(lib, gpu):
    import torch
    # first call: one GPU's share of ViT-L fc2 with 8 splits (16 MiB of partials);
    # second: a smaller GEMM with 4 splits that reuses the front of the scratch
    cases = [(512, 4096, 1024, 8, 80), (136, 2048, 256, 4, 81)]
    for M, K, N, splits, seed in cases:
        case = wl.random_24_f16(np.random.default_rng(seed), M, K, N)
        vals, meta = lib.w24_pack_f16(case["Wp"])
        A_d, v_d, m_d = T(case["A"]), T(vals), T(meta.view(np.int32))
        C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        rc = _static_call(lib, A_d, v_d, m_d, C, splits)
        assert rc == 0, lib.load().ssg_last_error().decode()
        got = H(C)
        ref = H(lib.w24_gemm_f16_splitk(A_d, v_d, m_d, splits))
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), (M, K, N, splits)
        C_ref, _ = oracle.ref_gemm_f16(case["A"], case["Wp"])
        assert oracle.loose_err(got, C_ref) <= 1e-2
        assert oracle.strict_ok_f16(got, C_ref, oracle.ref_abs_gemm(case["A"], case["Wp"]), K // 2)


def test_static_scratch_exact_integers(lib, gpu):
    """Exact integers: bit-exact against the oracle (every partial is an exact integer)."""
    case = wl.exact_int_24_f16(np.random.default_rng(82), 256, 4096, 512)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16_splitk_static(T(case["A"]), T(vals), T(meta.view(np.int32)), 8))
    _, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
    assert np.array_equal(C.view(np.uint16), C16.view(np.uint16))


def test_static_scratch_rejects_oversize(lib, gpu):
    """More partials than the scratch holds: a clear error, nothing launched."""
    import torch
    M, K, N = 4096, 4096, 1024  # 8 splits x 16 MiB > 32 MiB
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    vals = torch.zeros((N, K // 2), dtype=torch.float16, device="cuda")
    meta = torch.zeros((N, K // 32), dtype=torch.int32, device="cuda")
    with pytest.raises(lib.SsgError, match="static"):
        lib.w24_gemm_f16_splitk_static(A, vals, meta, 8)
