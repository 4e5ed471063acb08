"""Tile-wise GEMM under SSG_TW_NARROW (every tile keeps at most 64 columns).

The narrow-tile configurations size their stage buffers and registers for 64
kept columns: a 32-row-stage form with four workgroups per CU, and a
64-row-stage form for launches of at most two work items per CU.  Both run
the same matrix instructions over the same k order as the general kernel, so
the output must be bit-identical to the call without the flag, and it is
checked against the oracle (loose and strict bounds, or bit-exact on
exact-integer inputs) at the BERT-large FFN shapes of the tile-wise slides
("Accelerating Sparse DNN Models without Hardware-Support via Tile-Wise
Sparsity", the BERT results), on shapes with ragged token tails, and with the
transposed output.  A tile wider than 64 columns under the flag must come out
as quiet NaN in its whole window.
"""

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

NAN16 = 0x7E00
N_CUS = 256


def T(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def H(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def tw_terms(Wp, G):
    packed = oracle.ref_tw_pack(Wp, G)
    return np.repeat(np.maximum(np.diff(packed["k_ptr"]), 1), G).astype(np.float64)


def nan_out(torch, shape):
    return torch.full(shape, float("nan"), dtype=torch.float16, device="cuda")


def run_both(lib, A, Wp, G, out_t=False, At=None):
    """(narrow, general) outputs of the same call, each into a NaN-prefilled buffer."""
    import torch
    packed = lib.tw_pack_f16(Wp, G).to("cuda")
    At = T(np.ascontiguousarray(A.T)) if At is None else At  # (any M; the transpose kernel takes M % 8 == 0)
    M, N = A.shape[0], Wp.shape[1]
    shape = (N, M) if out_t else (M, N)
    Cn = H(lib.tw_gemm_f16_ex(At, packed, out_t=out_t, narrow=True, out=nan_out(torch, shape)))
    Cg = H(lib.tw_gemm_f16_ex(At, packed, out_t=out_t, narrow=False, out=nan_out(torch, shape)))
    return (Cn.T.copy(), Cg.T.copy()) if out_t else (Cn, Cg), packed


def items(M, T_):
    return (M + 127) // 128 * T_


# token tails (M % 8 != 0 gathers through registers), one item, few and many items
SHAPES = [(1, 256, 256, 128, [0.1, 0.2]), (17, 300, 256, 64, [0.5, 0.9, 0.2, 1.0]),
          (129, 512, 384, 128, [0.05, 0.25, 0.15]), (200, 96, 128, 32, [1.0, 0.0, 0.5, 0.3]),
          (256, 768, 512, 128, [0.1, 0.2, 0.25, 0.02]), (4096 + 136, 512, 1024, 128, 0.1),
          (8192 + 8, 256, 1024, 64, 0.3), (1024, 2048, 512, 128, [0.05, 0.1, 0.2, 0.15]),
          (264, 4096, 256, 64, [0.1, 0.3, 0.02, 0.5])]


def deep_form(M, K, N, G):
    return items(M, N // G) <= 2 * N_CUS and M % 8 == 0 and K >= 2048


def test_shapes_cover_both_narrow_forms():
    deep = [deep_form(M, K, N, G) for M, K, N, G, d in SHAPES]
    assert any(deep) and not all(deep)


@pytest.mark.parametrize("M,K,N,G,d", SHAPES)
def test_narrow_matches_general_and_oracle(lib, gpu, M, K, N, G, d):
    case = wl.random_tw_f16(np.random.default_rng(M + K + N + G), M, K, N, G, d)
    (Cn, Cg), packed = run_both(lib, case["A"], case["Wp"], G)
    assert packed.narrow() and packed.max_nt <= 64
    assert np.array_equal(Cn.view(np.uint16), Cg.view(np.uint16)), "narrow differs from the general kernel"
    C_ref, _ = oracle.ref_gemm_f16(case["A"], case["Wp"])
    assert oracle.loose_err(Cn, C_ref) <= 1e-2
    assert oracle.strict_ok_f16(Cn, C_ref, oracle.ref_abs_gemm(case["A"], case["Wp"]), tw_terms(case["Wp"], G))


@pytest.mark.parametrize("M,K,N,G,d", SHAPES[:5])
def test_narrow_transposed_output(lib, gpu, M, K, N, G, d):
    case = wl.random_tw_f16(np.random.default_rng(2 * M + K + G), M, K, N, G, d)
    (Cnt, Cgt), _ = run_both(lib, case["A"], case["Wp"], G, out_t=True)
    (Cn, _), _ = run_both(lib, case["A"], case["Wp"], G)
    assert np.array_equal(Cnt.view(np.uint16), Cgt.view(np.uint16))
    assert np.array_equal(Cnt.view(np.uint16), Cn.view(np.uint16))


@pytest.mark.parametrize("M,K,N,G,d", [(17, 300, 256, 64, [0.5, 0.9, 0.2, 1.0]),
                                       (136, 512, 384, 128, [0.05, 0.2, 0.1]),
                                       (2048, 640, 512, 128, [0.2, 0.1, 0.15, 0.05]),
                                       (6000, 320, 2048, 128, 0.2),  # 752 items: the four-per-CU form
                                       (512, 2048, 256, 64, [0.02, 0.01, 0.02, 0.015])])  # 64-row stages
def test_narrow_exact_integers(lib, gpu, M, K, N, G, d):
    ex = wl.exact_int_tw_f16(np.random.default_rng(M + 7), M, K, N, G, d)
    assert np.diff(oracle.ref_tw_pack(ex["Wp"], G)["k_ptr"]).max() <= 341  # every partial sum stays exact
    (Cn, _), _ = run_both(lib, ex["A"], ex["Wp"], G)
    _, C16 = oracle.ref_gemm_f16(ex["A"], ex["Wp"])
    assert np.array_equal(Cn.view(np.uint16), C16.view(np.uint16))
    (Cnt, _), _ = run_both(lib, ex["A"], ex["Wp"], G, out_t=True)
    assert np.array_equal(Cnt.view(np.uint16), C16.view(np.uint16))


@pytest.mark.parametrize("which", ["fc1", "fc2"])
def test_narrow_bert_large_ffn(lib, gpu, which):
    # fc1: 1536 items (the four-per-CU form); fc2: 384 items (64-row stages)
    c = wl.make_bert_large_ffn_tw()[which]
    assert deep_form(c["M"], c["K"], c["N"], c["G"]) == (which == "fc2")
    (Cn, Cg), packed = run_both(lib, c["A"], c["Wp"], c["G"])
    assert packed.max_nt == 40
    assert np.array_equal(Cn.view(np.uint16), Cg.view(np.uint16))
    C_ref, _ = oracle.ref_gemm_f16(c["A"], c["Wp"])
    n = tw_terms(c["Wp"], c["G"])
    assert oracle.loose_err(Cn, C_ref) <= 1e-2
    assert oracle.strict_ok_f16(Cn, C_ref, oracle.ref_abs_gemm(c["A"], c["Wp"]), n)


def test_narrow_row_major_a(lib, gpu):
    case = wl.random_tw_f16(np.random.default_rng(31), 136, 384, 256, 64, [0.3, 0.6, 0.1, 0.9])
    import torch
    packed = lib.tw_pack_f16(case["Wp"], 64).to("cuda")
    Cr = H(lib.tw_gemm_f16_ex(T(case["A"]), packed, a_rowmajor=True, narrow=True,
                              out=nan_out(torch, (136, 256))))
    Cg = H(lib.tw_gemm_f16_ex(T(case["A"]), packed, a_rowmajor=True, narrow=False))
    assert np.array_equal(Cr.view(np.uint16), Cg.view(np.uint16))
    C_ref, _ = oracle.ref_gemm_f16(case["A"], case["Wp"])
    assert oracle.loose_err(Cr, C_ref) <= 1e-2


@pytest.mark.parametrize("M,K", [(64, 2048), (64, 256), (5504 + 8, 256)])  # 64-row stages; four per CU
def test_narrow_flag_with_a_wide_tile_gives_nan_window(lib, gpu, M, K):
    # tile 1 keeps 128 columns (density 1.0) although the caller promises <= 64:
    # its whole window is NaN; the narrow tiles around it are computed normally
    import torch
    G, N = 128, 12 * 128
    case = wl.random_tw_f16(np.random.default_rng(M), M, K, N, G, [0.1, 1.0] + [0.2] * 10)
    packed = lib.tw_pack_f16(case["Wp"], G)
    assert np.diff(packed.n_ptr).tolist()[1] == 128
    dp = packed.to("cuda")
    At = lib.ssg_transpose_f16(T(case["A"]))
    C = H(lib.tw_gemm_f16_ex(At, dp, narrow=True, out=torch.zeros((M, N), dtype=torch.float16, device="cuda")))
    assert (C[:, G:2 * G].view(np.uint16) == NAN16).all()
    Cg = H(lib.tw_gemm_f16_ex(At, dp, narrow=False))
    keep = np.r_[0:G, 2 * G:N]
    assert np.array_equal(C[:, keep].view(np.uint16), Cg[:, keep].view(np.uint16))
    Ct = H(lib.tw_gemm_f16_ex(At, dp, narrow=True, out_t=True,
                              out=torch.zeros((N, M), dtype=torch.float16, device="cuda")))
    assert (Ct[G:2 * G].view(np.uint16) == NAN16).all()
    assert np.array_equal(Ct[keep].view(np.uint16), Cg[:, keep].T.view(np.uint16))


def test_narrow_flag_ignored_for_wide_tiles(lib, gpu):
    # G = 256 runs the wide configuration whatever the flag says
    case = wl.random_tw_f16(np.random.default_rng(5), 72, 256, 512, 256, [0.05, 0.04])
    (Cn, Cg), packed = run_both(lib, case["A"], case["Wp"], 256)
    assert packed.max_nt <= 64
    assert np.array_equal(Cn.view(np.uint16), Cg.view(np.uint16))
    C_ref, _ = oracle.ref_gemm_f16(case["A"], case["Wp"])
    assert oracle.loose_err(Cn, C_ref) <= 1e-2


def test_default_binding_takes_narrow_path_only_for_narrow_packs(lib, gpu):
    narrow = lib.tw_pack_f16(wl.random_tw_f16(np.random.default_rng(1), 8, 64, 256, 128, 0.1)["Wp"], 128)
    wide = lib.tw_pack_f16(wl.random_tw_f16(np.random.default_rng(1), 8, 64, 256, 128, 0.9)["Wp"], 128)
    assert narrow.narrow() and narrow.to("cuda").narrow()
    assert not wide.narrow() and not wide.to("cuda").narrow()
