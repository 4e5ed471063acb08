"""Split-K GEMMs (K cut into ranges run by separate workgroups, partial
accumulators summed by a second kernel) vs the oracle and vs the unsplit
kernels, through the C ABI.

Bars: int8 kinds bit-exact (the int32 sum of the partials is the
accumulator itself), for every output kind, equal to the unsplit call and to
the oracle; fp16 kinds within the strict per-element bound (fp32 summation
in another order), and bit-exact on exact-integer inputs.  Shapes include
one GPU's share of ViT-Large under 8-way token sharding (M = 512), where the
library splits on its own.
"""

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


def _check_f16(C, A, Wp, what, dense=False):
    """Loose and strict bounds; the strict one counts the products each output
    sums over all splits: K for the dense kinds, K/2 kept slots for 2:4."""
    C_ref, _ = oracle.ref_gemm_f16(A, Wp)
    n_terms = Wp.shape[0] if dense else Wp.shape[0] // 2
    assert oracle.loose_err(C, C_ref) <= 1e-2, what
    assert oracle.strict_ok_f16(C, C_ref, oracle.ref_abs_gemm(A, Wp), n_terms), what


def _exact_f16(C, A, Wp, what):
    _, C16 = oracle.ref_gemm_f16(A, Wp)
    assert np.array_equal(C.view(np.uint16), C16.view(np.uint16)), what


# K = 2048 fp16: 32 K stages
F16_SPLITS = [2, 4, 8, 32]


@pytest.mark.parametrize("splits", F16_SPLITS)
def test_w24_f16_splitk_random(lib, gpu, splits):
    case = wl.random_24_f16(np.random.default_rng(splits), 300, 2048, 256)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16_splitk(T(case["A"]), T(vals), T(meta.view(np.int32)), splits))
    _check_f16(C, case["A"], case["Wp"], f"w24 f16 splits={splits}")


@pytest.mark.parametrize("splits", F16_SPLITS)
def test_dense_f16_splitk_random(lib, gpu, splits):
    case = wl.random_24_f16(np.random.default_rng(10 + splits), 300, 2048, 256)
    C = H(lib.dense_gemm_f16_splitk(T(case["A"]), T(case["W"].T), splits))
    _check_f16(C, case["A"], case["W"], f"dense f16 splits={splits}", dense=True)


@pytest.mark.parametrize("splits", [2, 5])  # K = 640: 10 K stages
def test_f16_splitk_exact_integers(lib, gpu, splits):
    # every partial and every sum of partials is an exact integer below 2^24
    case = wl.exact_int_24_f16(np.random.default_rng(20 + splits), 129, 640, 192)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16_splitk(T(case["A"]), T(vals), T(meta.view(np.int32)), splits))
    _exact_f16(C, case["A"], case["Wp"], f"w24 f16 exact splits={splits}")


@pytest.mark.parametrize("out", ["i32", "f32", "f16", "i8"])
@pytest.mark.parametrize("splits", [2, 4, 8])
def test_w24_i8_splitk_bit_exact(lib, gpu, out, splits):
    rng = np.random.default_rng(30 + splits)
    case = wl.random_24_i8(rng, 200, 1024, 320)
    bias = None if out == "i32" else rng.normal(0, 4, 320).astype(np.float32)
    scale = None if out == "i32" else case["scale"]
    vals, meta = lib.w24_pack_i8(case["Wp"])
    args = (T(case["A"]), T(vals), T(meta.view(np.int32)), None if scale is None else T(scale),
            None if bias is None else T(bias))
    C = H(lib.w24_gemm_i8_splitk(*args, out_type=out, splits=splits))
    C1 = H(lib.w24_gemm_i8_out(*args, out_type=out, splits=1))
    assert np.array_equal(C.view(np.uint8), C1.view(np.uint8)), "differs from the unsplit kernel"
    acc = oracle.ref_acc_i8(case["A"], case["Wp"])
    ref = acc if out == "i32" else oracle.ref_i8_epilogue(acc, scale, bias, out)
    assert np.array_equal(C.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


@pytest.mark.parametrize("out", ["i32", "f32", "i8"])
def test_dense_i8_splitk_bit_exact(lib, gpu, out):
    rng = np.random.default_rng(40)
    case = wl.random_24_i8(rng, 136, 2048, 256)
    scale = None if out == "i32" else case["scale"]
    Wt = T(case["W"].T)
    C = H(lib.dense_gemm_i8_splitk(T(case["A"]), Wt, None if scale is None else T(scale), None, out_type=out,
                                   splits=4))
    acc = oracle.ref_acc_i8(case["A"], case["W"])
    ref = acc if out == "i32" else oracle.ref_i8_epilogue(acc, scale, None, out)
    assert np.array_equal(C.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


def test_i8_splitk_extreme_values(lib, gpu):
    # |acc| > 2^24 and sign changes between partials: the int32 sum stays exact
    M, K, N = 16, 4096, 64
    A = np.full((M, K), 127, np.int8)
    A[1::2] = -127
    Wp = np.zeros((K, N), np.int8)
    Wp[0::4] = 127
    Wp[3::4] = -127
    Wp[3::4, ::3] = 127
    Wp[: K // 2, 1::5] = -Wp[: K // 2, 1::5]
    scale = np.random.default_rng(6).uniform(1e-3, 1e-2, N).astype(np.float32)
    vals, meta = lib.w24_pack_i8(Wp)
    for splits in (2, 8, 32):
        C = H(lib.w24_gemm_i8(T(A), T(vals), T(meta.view(np.int32)), T(scale), splits=splits))
        assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(A, Wp, scale).view(np.uint32)), splits


@pytest.mark.parametrize("gname", ["qkv", "proj", "fc1", "fc2"])
def test_vit_large_shard8_default_split(lib, gpu, gname):
    """One GPU's share (M = 512) of the ViT-L layer, through the default entry points
    (the library picks the split); fp16 within the bound, int8 bit-exact."""
    M8 = wl.VIT_LARGE_M // 8
    for g in wl.vit_large_layers("f16", layers=1, M=M8):
        if g["name"].endswith(gname):
            vals, meta = lib.w24_pack_f16(g["Wp"])
            C = H(lib.w24_gemm_f16(T(g["A"]), T(vals), T(meta.view(np.int32))))
            _check_f16(C, g["A"], g["Wp"], g["name"])
    for g in wl.vit_large_layers("i8", layers=1, M=M8):
        if g["name"].endswith(gname):
            vals, meta = lib.w24_pack_i8(g["Wp"])
            C = H(lib.w24_gemm_i8(T(g["A"]), T(vals), T(meta.view(np.int32)), T(g["scale"])))
            assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(g["A"], g["Wp"], g["scale"]).view(np.uint32))


def test_splitk_workspace_reused_across_calls(lib, gpu):
    """A caller workspace reused by back-to-back split calls on one stream (stream order)."""
    import torch
    rng = np.random.default_rng(50)
    cases = [wl.random_24_i8(rng, 96, 2048, 128) for _ in range(3)]
    ws = torch.empty(lib.splitk_workspace_bytes(96, 128, 8), dtype=torch.uint8, device="cuda")
    outs = []
    for c in cases:
        vals, meta = lib.w24_pack_i8(c["Wp"])
        outs.append(lib.w24_gemm_i8_splitk(T(c["A"]), T(vals), T(meta.view(np.int32)), T(c["scale"]), None,
                                           out_type="f32", splits=8, workspace=ws))
    for c, o in zip(cases, outs):
        assert np.array_equal(H(o).view(np.uint32), oracle.ref_gemm_i8(c["A"], c["Wp"], c["scale"]).view(np.uint32))


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_f16_split_tiles_of_a_shard(lib, gpu, splits):
    """One GPU's share of ViT-L fc2 (512 x 4096 x 1024) with each split count:
    the split launch takes 64 x 64 (2), 64 x 128 (4) or 128 x 128 (8) tiles;
    2:4 and dense fp16 within the bound."""
    case = wl.random_24_f16(np.random.default_rng(60 + splits), 512, 4096, 1024)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16_splitk(T(case["A"]), T(vals), T(meta.view(np.int32)), splits))
    _check_f16(C, case["A"], case["Wp"], f"w24 f16 shard fc2 splits={splits}")
    C = H(lib.dense_gemm_f16_splitk(T(case["A"]), T(case["W"].T), splits))
    _check_f16(C, case["A"], case["W"], f"dense f16 shard fc2 splits={splits}", dense=True)


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_f16_split_tiles_of_a_shard_exact(lib, gpu, splits):
    """The same split forms (64 x 64 x 2, 64 x 128 x 4, 128 x 128 x 8) on
    exact-integer inputs: every fp32 partial and their sum are exact integers,
    so the one fp16 rounding matches the oracle's bit for bit (|C| stays far
    below the fp16 range: at most 4096 * 3 * 2)."""
    case = wl.exact_int_24_f16(np.random.default_rng(70 + splits), 512, 4096, 1024)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16_splitk(T(case["A"]), T(vals), T(meta.view(np.int32)), splits))
    _exact_f16(C, case["A"], case["Wp"], f"w24 f16 shard fc2 exact splits={splits}")
    C = H(lib.dense_gemm_f16_splitk(T(case["A"]), T(case["W"].T), splits))
    _exact_f16(C, case["A"], case["W"], f"dense f16 shard fc2 exact splits={splits}")
