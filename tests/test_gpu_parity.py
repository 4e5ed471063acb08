"""HIP kernels vs the oracle, element by element, through the C ABI.

Bars (from the arithmetic; see oracle/bounds.py):
* int8 / int32 paths: bit-exact (int32 accumulators and fp32 scaled outputs);
* fp16 paths: max|C - C_ref| <= 1e-2 * max|C_ref| (acceptance) and the strict
  per-element bound |C - C_ref| <= 2^-11 |C_ref| + 2^-25 + 2 n 2^-24 S;
* exact-integer inputs and one-hot weights: bit-exact for fp16 too (every fp32
  partial sum is an exact integer, so the single fp16 rounding is the
  oracle's round-to-nearest-even of the exact value);
* transpose: bit-exact.
Shapes span several tiles with ragged token tails (M = 1, 17, 200, ...).
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


def meta_t(meta):
    return T(meta.view(np.int32))


def run_w24_f16(lib, A, Wp, out=None):
    vals, meta = lib.w24_pack_f16(Wp)
    return H(lib.w24_gemm_f16(T(A), T(vals), meta_t(meta), out=out))


def run_w24_i8(lib, A, Wp, scale):
    vals, meta = lib.w24_pack_i8(Wp)
    return H(lib.w24_gemm_i8(T(A), T(vals), meta_t(meta), None if scale is None else T(scale)))


def tw_terms(Wp, G):
    """Products each output column sums in the tile-wise kernel: K_t of its
    tile (the kernel walks only the tile's kept rows), one entry per column."""
    packed = oracle.ref_tw_pack(Wp, G)
    return np.repeat(np.maximum(np.diff(packed["k_ptr"]), 1), G).astype(np.float64)


def check_f16(C, A, Wp, n_terms, what=""):
    """n_terms: products summed per output (a number, or one per column)."""
    C_ref, _ = oracle.ref_gemm_f16(A, Wp)
    S = oracle.ref_abs_gemm(A, Wp)
    err = oracle.loose_err(C, C_ref)
    assert err <= 1e-2, f"{what}: loose error {err}"
    assert oracle.strict_ok_f16(C, C_ref, S, n_terms), f"{what}: strict bound violated"


def check_f16_exact(C, A, Wp, what=""):
    _, C16 = oracle.ref_gemm_f16(A, Wp)
    bad = np.flatnonzero(C.view(np.uint16) != C16.view(np.uint16))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {np.unravel_index(bad[0], C.shape)}"


SMALL = [(1, 64, 64), (17, 128, 256), (200, 512, 320), (129, 256, 64), (64, 192, 128)]


# ---------------------------------------------------------------- 2:4 fp16
@pytest.mark.parametrize("M,K,N", SMALL)
def test_w24_f16_random(lib, gpu, M, K, N):
    case = wl.random_24_f16(np.random.default_rng(M * 7 + K), M, K, N)
    C = run_w24_f16(lib, case["A"], case["Wp"])
    check_f16(C, case["A"], case["Wp"], K // 2, f"w24 f16 {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", SMALL + [(300, 1024, 256)])
def test_w24_f16_exact_integers(lib, gpu, M, K, N):
    case = wl.exact_int_24_f16(np.random.default_rng(K + N), M, K, N)
    check_f16_exact(run_w24_f16(lib, case["A"], case["Wp"]), case["A"], case["Wp"], "w24 f16 exact")


def test_w24_f16_one_hot(lib, gpu):
    case = wl.one_hot_24(np.random.default_rng(3), 77, 256, 192)
    C = run_w24_f16(lib, case["A"], case["Wp"])
    assert np.array_equal(C.view(np.uint16), case["A"][:, case["k_of_n"]].view(np.uint16))


def test_w24_f16_every_position_pair(lib, gpu):
    # Each column walks all six position pairs across its groups, with exact integers.
    M, K, N = 40, 384, 64
    rng = np.random.default_rng(4)
    A = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    Wp = np.zeros((K, N), np.float16)
    pairs = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]
    for n in range(N):
        for g in range(K // 4):
            p0, p1 = pairs[(g + n) % 6]
            Wp[4 * g + p0, n] = rng.integers(1, 3) * (1 if (g + n) % 2 else -1)
            Wp[4 * g + p1, n] = rng.integers(-2, 3)
    check_f16_exact(run_w24_f16(lib, A, Wp), A, Wp, "position pairs")


def test_w24_f16_small(lib, gpu):
    c = wl.make_small_w24_f16()
    check_f16(run_w24_f16(lib, c["A"], c["Wp"]), c["A"], c["Wp"], c["K"] // 2, c["name"])


@pytest.mark.parametrize("gname", ["qkv", "proj", "fc1", "fc2"])
def test_w24_f16_vit_large_layer0(lib, gpu, gname):
    for g in wl.vit_large_layers("f16", layers=1):
        if g["name"].endswith(gname):
            check_f16(run_w24_f16(lib, g["A"], g["Wp"]), g["A"], g["Wp"], g["K"] // 2, g["name"])


# ---------------------------------------------------------------- 2:4 int8
@pytest.mark.parametrize("M,K,N", [(1, 128, 64), (17, 256, 256), (200, 768, 320), (129, 512, 64)])
@pytest.mark.parametrize("scaled", [False, True])
def test_w24_i8_bit_exact(lib, gpu, M, K, N, scaled):
    case = wl.random_24_i8(np.random.default_rng(M + K + N), M, K, N)
    scale = case["scale"] if scaled else None
    C = run_w24_i8(lib, case["A"], case["Wp"], scale)
    ref = oracle.ref_gemm_i8(case["A"], case["Wp"], scale)
    assert C.dtype == ref.dtype
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


def test_w24_i8_one_hot(lib, gpu):
    case = wl.one_hot_24(np.random.default_rng(5), 65, 256, 128, dtype=np.int8)
    C = run_w24_i8(lib, case["A"], case["Wp"], None)
    assert np.array_equal(C, case["A"][:, case["k_of_n"]].astype(np.int32))


def test_w24_i8_extreme_values(lib, gpu):
    # +-127 everywhere, K = 4096: |acc| = 2048 * 127^2 > 2^24 exercises int32 range and fp32 rounding.
    M, K, N = 16, 4096, 64
    A = np.full((M, K), 127, np.int8)
    A[1::2] = -127
    Wp = np.zeros((K, N), np.int8)
    Wp[0::4] = 127
    Wp[3::4] = -127
    Wp[3::4, ::3] = 127
    scale = np.random.default_rng(6).uniform(1e-3, 1e-2, N).astype(np.float32)
    for s in (None, scale):
        C = run_w24_i8(lib, A, Wp, s)
        ref = oracle.ref_gemm_i8(A, Wp, s)
        assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


def test_w24_i8_vit_base_fc1(lib, gpu):
    c = wl.make_vit_base_fc1_i8()
    for s in (None, c["scale"]):
        C = run_w24_i8(lib, c["A"], c["Wp"], s)
        ref = oracle.ref_gemm_i8(c["A"], c["Wp"], s)
        assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


def test_i8_large_tile_path(lib, gpu):
    # K > 1024 with many tiles selects the 256 x 256 eight-wave kernels.
    case = wl.random_24_i8(np.random.default_rng(14), 4096, 2048, 3072)
    C = run_w24_i8(lib, case["A"], case["Wp"], case["scale"])
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"]).view(np.uint32))
    Cd = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), None))
    assert np.array_equal(Cd, oracle.ref_gemm_i8(case["A"], case["W"]))


# Short-K int8 tile choice: (M, K, N) -> sparse tile / dense tile.  Ragged M
# (not a multiple of 128) so every path also runs a partial last tile row.
I8_SHORT_K_PATHS = [
    (4000, 512, 4096),   # 512 Mid tiles -> sparse 128x256; 256 Big tiles -> dense 256x256
    (3000, 768, 2048),   # 192 Mid tiles -> sparse 128x128 two-stage; 96 Big tiles -> dense 128x128
    (9000, 256, 3072),   # 852 Mid tiles -> sparse 128x128 two-stage; 432 Big tiles -> dense 256x256
]


@pytest.mark.parametrize("M,K,N", I8_SHORT_K_PATHS)
def test_i8_short_k_tile_paths(lib, gpu, M, K, N):
    case = wl.random_24_i8(np.random.default_rng(M + N), M, K, N)
    C = run_w24_i8(lib, case["A"], case["Wp"], case["scale"])
    ref = oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"])
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))
    Cd = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), T(case["scale"])))
    refd = oracle.ref_gemm_i8(case["A"], case["W"], case["scale"])
    assert np.array_equal(Cd.view(np.uint32), refd.view(np.uint32))


@pytest.mark.parametrize("gname", ["qkv", "fc2"])
def test_w24_i8_vit_large_layer0(lib, gpu, gname):
    for g in wl.vit_large_layers("i8", layers=1):
        if g["name"].endswith(gname):
            C = run_w24_i8(lib, g["A"], g["Wp"], g["scale"])
            ref = oracle.ref_gemm_i8(g["A"], g["Wp"], g["scale"])
            assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- dense baselines
@pytest.mark.parametrize("M,K,N", SMALL)
def test_dense_f16(lib, gpu, M, K, N):
    rng = np.random.default_rng(M + 3 * K)
    A = wl.f16_normal(rng, (M, K))
    W = wl.f16_normal(rng, (K, N), 0.02)
    C = H(lib.dense_gemm_f16(T(A), T(W.T)))
    check_f16(C, A, W, K, f"dense f16 {M}x{K}x{N}")
    ex = wl.exact_int_24_f16(rng, M, K, N)
    check_f16_exact(H(lib.dense_gemm_f16(T(ex["A"]), T(ex["W"].T))), ex["A"], ex["W"], "dense exact")


# The shapes where the dense fp16 kernel runs its 256 x 256 tile (two-stage
# ring) and is the denominator of the fp16 speedups: ViT-Large fc1 and the
# BERT-base FFN fc1 shape of the tile-wise workload.
DENSE_BIG = [(4096, 1024, 4096), (4096, 768, 3072)]


@pytest.mark.parametrize("M,K,N", DENSE_BIG)
def test_dense_f16_big_tile(lib, gpu, M, K, N):
    assert lib.tile_choice(lib.SSG_KIND_DENSE_F16, M, N, K) == (256, 256)
    rng = np.random.default_rng(M + 5 * K + N)
    A = wl.f16_normal(rng, (M, K))
    W = wl.f16_normal(rng, (K, N), 0.02)
    C = H(lib.dense_gemm_f16(T(A), T(W.T), splits=1))
    check_f16(C, A, W, K, f"dense f16 256x256 tile {M}x{K}x{N}")
    # exact integers: every fp32 partial sum is an exact integer (|C| <= 6K),
    # so the single fp16 rounding equals the oracle's bit for bit
    ex = wl.exact_int_24_f16(rng, M, K, N)
    check_f16_exact(H(lib.dense_gemm_f16(T(ex["A"]), T(ex["W"].T), splits=1)), ex["A"], ex["W"],
                    f"dense f16 256x256 tile exact {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(1, 128, 64), (200, 768, 320), (129, 512, 64)])
@pytest.mark.parametrize("scaled", [False, True])
def test_dense_i8(lib, gpu, M, K, N, scaled):
    case = wl.random_24_i8(np.random.default_rng(M * K), M, K, N)
    scale = case["scale"] if scaled else None
    C = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), None if scale is None else T(scale)))
    ref = oracle.ref_gemm_i8(case["A"], case["W"], scale)
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


def test_dense_equals_sparse_on_pruned_weight(lib, gpu):
    # Identity from the definition: the 2:4 result equals the dense GEMM on W_p (int8: bit-exact).
    case = wl.random_24_i8(np.random.default_rng(8), 96, 512, 256)
    Cs = run_w24_i8(lib, case["A"], case["Wp"], case["scale"])
    Cd = H(lib.dense_gemm_i8(T(case["A"]), T(case["Wp"].T), T(case["scale"])))
    assert np.array_equal(Cs.view(np.uint32), Cd.view(np.uint32))


# ---------------------------------------------------------------- int8 epilogues
def _bits(x):
    return x.view({4: np.uint32, 2: np.uint16, 1: np.uint8}[x.dtype.itemsize])


def _i8_out_case(rng, M, K, N, out):
    case = wl.random_24_i8(rng, M, K, N)
    # y in each output kind's working range: fp16 up to a few thousand, int8 around +-100
    scale = {"f32": case["scale"], "f16": case["scale"] * np.float32(20.0),
             "i8": rng.uniform(2e-4, 2e-3, size=N).astype(np.float32)}[out]
    bias = rng.normal(0, 4.0, size=N).astype(np.float32)
    return case, scale, bias


I8_OUT_SHAPES = [(1, 128, 64), (130, 768, 192), (257, 256, 320), (1000, 1024, 576)]


@pytest.mark.parametrize("out", ["f32", "f16", "i8"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M,K,N", I8_OUT_SHAPES)
def test_w24_i8_out_bit_exact(lib, gpu, M, K, N, out, with_bias):
    rng = np.random.default_rng(M * 7 + K + N)
    case, scale, bias = _i8_out_case(rng, M, K, N, out)
    b = bias if with_bias else None
    vals, meta = lib.w24_pack_i8(case["Wp"])
    C = H(lib.w24_gemm_i8_out(T(case["A"]), T(vals), meta_t(meta), T(scale), None if b is None else T(b),
                              out_type=out))
    ref = oracle.ref_gemm_i8_out(case["A"], case["Wp"], scale, b, out)
    assert C.dtype == ref.dtype
    bad = np.flatnonzero(_bits(C) != _bits(ref))
    assert bad.size == 0, f"{bad.size} mismatches, first at {np.unravel_index(bad[0], C.shape)}"


@pytest.mark.parametrize("out", ["i32", "f32", "f16", "i8"])
def test_dense_i8_out_bit_exact(lib, gpu, out):
    rng = np.random.default_rng(21)
    case, scale, bias = _i8_out_case(rng, 200, 512, 320, out if out != "i32" else "f32")
    s, b = (None, None) if out == "i32" else (scale, bias)
    C = H(lib.dense_gemm_i8_out(T(case["A"]), T(case["W"].T), None if s is None else T(s),
                                None if b is None else T(b), out_type=out))
    ref = oracle.ref_gemm_i8_out(case["A"], case["W"], s, b, out)
    assert np.array_equal(_bits(C), _bits(ref))


def test_i8_out_saturation_and_ties(lib, gpu):
    # small activations and weights with scale 0.5: odd accumulators are exact
    # ties (x.5, rounded to even), and two rows of +-127 drive outputs into saturation
    rng = np.random.default_rng(22)
    A = rng.integers(-2, 3, size=(64, 256)).astype(np.int8)
    A[0] = 127
    A[1] = -127
    Wp = wl.prune24_magnitude(rng.integers(-1, 2, size=(256, 64)).astype(np.int8))
    scale = np.full(64, 0.5, np.float32)
    acc = oracle.ref_acc_i8(A, Wp)
    assert (acc % 2 != 0).sum() > 500 and (np.abs(acc * 0.5) > 128).sum() > 20
    vals, meta = lib.w24_pack_i8(Wp)
    for out in ("i8", "f16"):
        C = H(lib.w24_gemm_i8_out(T(A), T(vals), meta_t(meta), T(scale), out_type=out))
        ref = oracle.ref_gemm_i8_out(A, Wp, scale, None, out)
        assert np.array_equal(_bits(C), _bits(ref)), out


@pytest.mark.parametrize("out", ["f16", "i8"])
def test_w24_i8_out_vit_base_fc1(lib, gpu, out):
    c = wl.make_vit_base_fc1_i8()
    rng = np.random.default_rng(5)
    scale = (c["scale"] * np.float32(0.02)) if out == "i8" else c["scale"]
    bias = rng.normal(0, 2.0, size=c["N"]).astype(np.float32)
    vals, meta = lib.w24_pack_i8(c["Wp"])
    C = H(lib.w24_gemm_i8_out(T(c["A"]), T(vals), meta_t(meta), T(scale), T(bias), out_type=out))
    ref = oracle.ref_gemm_i8_out(c["A"], c["Wp"], scale, bias, out)
    assert np.array_equal(_bits(C), _bits(ref))


# ---------------------------------------------------------------- tile-wise
def run_tw(lib, A, Wp, G, prefill_nan=True):
    import torch
    packed = lib.tw_pack_f16(Wp, G).to("cuda")
    At = lib.ssg_transpose_f16(T(A))
    out = torch.full((A.shape[0], Wp.shape[1]), float("nan"), dtype=torch.float16, device="cuda") \
        if prefill_nan else None
    return H(lib.tw_gemm_f16(At, packed, out=out))


TW_SMALL = [(8, 64, 32, 16, [0.5, 1.0]), (136, 200, 96, 32, [0.3, 0.0, 0.9]),
            (256, 768, 384, 128, [0.1, 0.25, 0.4]), (24, 1000, 64, 64, 0.6), (200, 96, 128, 128, 1.0)]


@pytest.mark.parametrize("M,K,N,G,d", TW_SMALL)
def test_tw_random(lib, gpu, M, K, N, G, d):
    case = wl.random_tw_f16(np.random.default_rng(M + K + G), M, K, N, G, d)
    C = run_tw(lib, case["A"], case["Wp"], G)
    packed = oracle.ref_tw_pack(case["Wp"], G)
    check_f16(C, case["A"], case["Wp"], tw_terms(case["Wp"], G), f"tw {M}x{K}x{N} G={G}")
    # pruned columns are exact +0
    kept = np.zeros(N, bool)
    for t in range(packed["T"]):
        kept[t * G + packed["offset_n"][packed["n_ptr"][t]:packed["n_ptr"][t + 1]]] = True
    assert (C[:, ~kept].view(np.uint16) == 0).all()


@pytest.mark.parametrize("M,K,N,G,d", TW_SMALL)
def test_tw_exact_integers(lib, gpu, M, K, N, G, d):
    case = wl.exact_int_tw_f16(np.random.default_rng(K), M, K, N, G, d)
    check_f16_exact(run_tw(lib, case["A"], case["Wp"], G), case["A"], case["Wp"], "tw exact")


def test_tw_one_hot(lib, gpu):
    case = wl.one_hot_tw(np.random.default_rng(9), 64, 512, 256, 128)
    C = run_tw(lib, case["A"], case["Wp"], 128)
    for n in range(256):
        if case["k_of_n"][n] >= 0:
            assert np.array_equal(C[:, n].view(np.uint16), case["A"][:, case["k_of_n"][n]].view(np.uint16))
        else:
            assert (C[:, n].view(np.uint16) == 0).all()


def test_tw_all_zero_weight(lib, gpu):
    A = wl.f16_normal(np.random.default_rng(10), (32, 64))
    C = run_tw(lib, A, np.zeros((64, 256), np.float16), 128)
    assert (C.view(np.uint16) == 0).all()


def test_tw_bert_base_fc1(lib, gpu):
    c = wl.make_bert_base_fc1_tw()
    C = run_tw(lib, c["A"], c["Wp"], c["G"])
    check_f16(C, c["A"], c["Wp"], tw_terms(c["Wp"], c["G"]), c["name"])


@pytest.mark.parametrize("which", ["fc1", "fc2"])
def test_tw_bert_large_ffn(lib, gpu, which):
    c = wl.make_bert_large_ffn_tw()[which]
    C = run_tw(lib, c["A"], c["Wp"], c["G"])
    n = tw_terms(c["Wp"], c["G"])
    assert n.max() == {"fc1": 328, "fc2": 1311}[which]  # K_t of the uniform 10 % tiles
    check_f16(C, c["A"], c["Wp"], n, c["name"])


def test_tw_indexed_oracle_agrees(lib, gpu):
    # The kernel against the slide's indexed formulation (not the masked dense one).
    case = wl.random_tw_f16(np.random.default_rng(11), 64, 256, 256, 128, [0.2, 0.5])
    C = run_tw(lib, case["A"], case["Wp"], 128)
    ref = oracle.ref_tw_gemm_indexed(case["A"], oracle.ref_tw_pack(case["Wp"], 128), 256, 128)
    assert oracle.loose_err(C, ref) <= 1e-2


# ---------------------------------------------------------------- block-wise through the tile-wise kernel
@pytest.mark.parametrize("b", [32, 64])
@pytest.mark.parametrize("d", [0.25, 0.5, 1.0])
def test_blockwise_via_tilewise_kernel(lib, gpu, b, d):
    # a b x b block-pruned weight (the slides' 32x32 and 64x64 block-sparse
    # patterns) is a tile-wise weight (G = b) of whole b-row runs
    rng = np.random.default_rng(50 + b)
    A = wl.f16_normal(rng, (200, 512))
    Wp = wl.prune_blockwise(wl.f16_normal(rng, (512, 256), 0.02), b, d)
    packed = lib.tw_pack_f16(Wp, b)
    assert (np.diff(packed.n_ptr) == b).all() and (np.diff(packed.k_ptr) % b == 0).all()
    C = run_tw(lib, A, Wp, b)
    check_f16(C, A, Wp, tw_terms(Wp, b), f"BW {b}x{b} d={d}")
    # exact integers: bit-exact
    Ax = rng.integers(-3, 4, size=(200, 512)).astype(np.float16)
    Wx = wl.prune_blockwise(rng.integers(-2, 3, size=(512, 256)).astype(np.float16), b, d)
    check_f16_exact(run_tw(lib, Ax, Wx, b), Ax, Wx, f"BW {b}x{b} d={d} exact")


# ---------------------------------------------------------------- int8 tile-wise
TW8_SHAPES = [(16, 64, 32, 16, [0.5, 1.0]), (144, 200, 96, 32, [0.3, 0.0, 0.9]),
              (256, 768, 384, 128, [0.1, 0.25, 0.4]), (48, 1000, 64, 64, 0.6), (208, 96, 128, 128, 1.0)]


def run_tw_i8(lib, A, Wp, G, scale, bias, out):
    packed = lib.tw_pack_i8(Wp, G).to("cuda")
    At = T(np.ascontiguousarray(A.T))
    return H(lib.tw_gemm_i8(At, packed, None if scale is None else T(scale), None if bias is None else T(bias),
                            out_type=out))


@pytest.mark.parametrize("out", ["i32", "f32", "f16", "i8"])
@pytest.mark.parametrize("M,K,N,G,d", TW8_SHAPES)
def test_tw_i8_bit_exact(lib, gpu, M, K, N, G, d, out):
    rng = np.random.default_rng(M + 5 * K + G)
    case = wl.random_tw_i8(rng, M, K, N, G, d)
    scale = {"i32": None, "f32": case["scale"], "f16": case["scale"] * np.float32(20.0),
             "i8": rng.uniform(2e-4, 2e-3, size=N).astype(np.float32)}[out]
    bias = None if out == "i32" else rng.normal(0, 3.0, size=N).astype(np.float32)
    C = run_tw_i8(lib, case["A"], case["Wp"], G, scale, bias, out)
    ref = oracle.ref_gemm_i8_out(case["A"], case["Wp"], scale, bias, out)
    bad = np.flatnonzero(_bits(C) != _bits(ref))
    assert bad.size == 0, f"{bad.size} mismatches, first at {np.unravel_index(bad[0], C.shape)}"


def test_tw_i8_no_bias_pruned_columns(lib, gpu):
    # without bias a pruned column is the epilogue of a zero accumulator: +0 for
    # positive scales
    rng = np.random.default_rng(40)
    case = wl.random_tw_i8(rng, 64, 256, 256, 128, [0.2, 0.5])
    C = run_tw_i8(lib, case["A"], case["Wp"], 128, case["scale"], None, "f32")
    ref = oracle.ref_gemm_i8_out(case["A"], case["Wp"], case["scale"], None, "f32")
    assert np.array_equal(_bits(C), _bits(ref))


@pytest.mark.parametrize("out", ["f16", "i8"])
def test_tw_i8_workload(lib, gpu, out):
    c = wl.make_bert_base_fc1_tw_i8()
    rng = np.random.default_rng(41)
    scale = c["scale"] if out == "f16" else (c["scale"] * np.float32(0.05))
    bias = rng.normal(0, 2.0, size=c["N"]).astype(np.float32)
    C = run_tw_i8(lib, c["A"], c["Wp"], c["G"], scale, bias, out)
    ref = oracle.ref_gemm_i8_out(c["A"], c["Wp"], scale, bias, out)
    assert np.array_equal(_bits(C), _bits(ref))


# ---------------------------------------------------------------- tile-wise: fused transpose, tile ranges, streams
def _tw_setup(lib, A, Wp, G):
    packed = lib.tw_pack_f16(Wp, G).to("cuda")
    At = lib.ssg_transpose_f16(T(A))
    return packed, At


@pytest.mark.parametrize("M,K,N,G,d", TW_SMALL)
def test_tw_transposed_output(lib, gpu, M, K, N, G, d):
    import torch
    case = wl.random_tw_f16(np.random.default_rng(M + 2 * K + G), M, K, N, G, d)
    packed, At = _tw_setup(lib, case["A"], case["Wp"], G)
    C = H(lib.tw_gemm_f16(At, packed))
    Ct = H(lib.tw_gemm_f16_ex(At, packed, out_t=True,
                              out=torch.full((N, M), float("nan"), dtype=torch.float16, device="cuda")))
    assert Ct.shape == (N, M)
    # the same products in the same order: bit-identical, only the layout differs
    assert np.array_equal(Ct.T.view(np.uint16), C.view(np.uint16))


@pytest.mark.parametrize("M,K,N,G,d", TW_SMALL)
def test_tw_row_major_a(lib, gpu, M, K, N, G, d):
    # the "without transpose" case reads A [M][K] directly; the LDS stage holds the
    # same values in the same places, so the result is bit-identical
    case = wl.random_tw_f16(np.random.default_rng(M + 3 * K + G), M, K, N, G, d)
    packed, At = _tw_setup(lib, case["A"], case["Wp"], G)
    C = H(lib.tw_gemm_f16(At, packed))
    Cr = H(lib.tw_gemm_f16_ex(T(case["A"]), packed, a_rowmajor=True))
    check_f16(Cr, case["A"], case["Wp"], tw_terms(case["Wp"], G), f"tw row-major A {M}x{K}x{N}")
    assert np.array_equal(Cr.view(np.uint16), C.view(np.uint16))
    Crt = H(lib.tw_gemm_f16_ex(T(case["A"]), packed, a_rowmajor=True, out_t=True))
    assert np.array_equal(Crt.T.view(np.uint16), C.view(np.uint16))
    # exact integers through the row-major gather: bit-exact against the oracle
    ex = wl.exact_int_tw_f16(np.random.default_rng(M + K), M, K, N, G, d)
    px = lib.tw_pack_f16(ex["Wp"], G).to("cuda")
    check_f16_exact(H(lib.tw_gemm_f16_ex(T(ex["A"]), px, a_rowmajor=True)), ex["A"], ex["Wp"], "tw row-major exact")


def test_tw_chain_without_transpose(lib, gpu):
    # two tile-wise layers: layer 1 writes Ct1 [N1][M], which is layer 2's At directly
    rng = np.random.default_rng(30)
    M, K, N1, N2, G = 256, 384, 512, 256, 128
    l1 = wl.random_tw_f16(rng, M, K, N1, G, [0.3, 0.5, 0.2, 0.4])
    W2 = wl.prune_tilewise(wl.f16_normal(rng, (N1, N2), 0.05), G, np.array([0.4, 0.25]))
    p1 = lib.tw_pack_f16(l1["Wp"], G).to("cuda")
    p2 = lib.tw_pack_f16(W2, G).to("cuda")
    Ct1 = lib.tw_gemm_f16_ex(lib.ssg_transpose_f16(T(l1["A"])), p1, out_t=True)
    C2 = H(lib.tw_gemm_f16(Ct1, p2))
    A2 = H(Ct1).T.copy()  # layer 1's fp16 output, as the oracle's input of layer 2
    check_f16(A2, l1["A"], l1["Wp"], tw_terms(l1["Wp"], G), "chain layer 1")
    check_f16(C2, A2, W2, tw_terms(W2, G), "chain layer 2")


def test_tw_tile_ranges(lib, gpu):
    import torch
    case = wl.random_tw_f16(np.random.default_rng(31), 200, 512, 640, 128, [0.2, 0.5, 0.0, 0.8, 0.3])
    packed, At = _tw_setup(lib, case["A"], case["Wp"], 128)
    full = H(lib.tw_gemm_f16(At, packed))
    check_f16(full, case["A"], case["Wp"], tw_terms(case["Wp"], 128), "tw tile ranges, grouped launch")
    C = torch.full((200, 640), float("nan"), dtype=torch.float16, device="cuda")
    lib.tw_gemm_f16_ex(At, packed, t_first=1, t_count=2, out=C)
    part = H(C)
    order = H(packed.tile_order)
    done = set(int(t) for t in order[1:3])
    for t in range(5):
        win = part[:, t * 128:(t + 1) * 128]
        if t in done:
            assert np.array_equal(win.view(np.uint16), full[:, t * 128:(t + 1) * 128].view(np.uint16))
        else:
            assert np.isnan(win).all()  # tiles outside the range are not written
    lib.tw_gemm_f16_ex(At, packed, t_first=0, t_count=1, out=C)
    lib.tw_gemm_f16_ex(At, packed, t_first=3, t_count=2, out=C)
    assembled = H(C)
    check_f16(assembled, case["A"], case["Wp"], tw_terms(case["Wp"], 128), "tw tile ranges, assembled")
    assert np.array_equal(assembled.view(np.uint16), full.view(np.uint16))
    # exact integers, assembled from three ranges: bit-exact against the oracle
    ex = wl.exact_int_tw_f16(np.random.default_rng(32), 200, 512, 640, 128, [0.2, 0.5, 0.0, 0.8, 0.3])
    px, Atx = _tw_setup(lib, ex["A"], ex["Wp"], 128)
    Cx = torch.full((200, 640), float("nan"), dtype=torch.float16, device="cuda")
    for t0, tc in ((3, 2), (0, 1), (1, 2)):
        lib.tw_gemm_f16_ex(Atx, px, t_first=t0, t_count=tc, out=Cx)
    check_f16_exact(H(Cx), ex["A"], ex["Wp"], "tw tile ranges exact")


def test_tw_multi_stream_schedule(lib, gpu):
    import torch
    c = wl.make_bert_base_fc1_tw()
    packed, At = _tw_setup(lib, c["A"], c["Wp"], c["G"])
    full = H(lib.tw_gemm_f16(At, packed))
    streams = [torch.cuda.Stream() for _ in range(4)]
    C = H(lib.tw_gemm_f16_streams(At, packed, streams))
    check_f16(C, c["A"], c["Wp"], tw_terms(c["Wp"], c["G"]), "tw multi-stream schedule")
    assert np.array_equal(C.view(np.uint16), full.view(np.uint16))
    # exact integers over the streams: bit-exact against the oracle
    ex = wl.exact_int_tw_f16(np.random.default_rng(33), 512, 768, 1536, 128,
                             np.linspace(0.05, 0.6, 12))
    px, Atx = _tw_setup(lib, ex["A"], ex["Wp"], 128)
    check_f16_exact(H(lib.tw_gemm_f16_streams(Atx, px, streams)), ex["A"], ex["Wp"], "tw streams exact")


# ---------------------------------------------------------------- tile-wise limits: any M >= 1, tiles up to 256 columns
# (M, K, N, G, densities): token counts that are not multiples of 8 or 16 (the
# K-major At is then gathered through registers) and 256-column tiles (the
# wide configuration), alone and together
TW_LIMITS = [(1, 256, 512, 256, [0.3, 0.7]), (17, 300, 256, 128, [0.5, 0.2]),
             (129, 512, 768, 256, [0.1, 0.4, 1.0]), (7, 64, 64, 32, [0.5, 1.0]),
             (200, 384, 512, 256, [0.25, 0.9]), (136, 200, 512, 256, [0.6, 0.0])]


def _at(A):
    return T(np.ascontiguousarray(A.T))


@pytest.mark.parametrize("M,K,N,G,d", TW_LIMITS)
def test_tw_limits_f16(lib, gpu, M, K, N, G, d):
    import torch
    case = wl.random_tw_f16(np.random.default_rng(M * 3 + K + G), M, K, N, G, d)
    packed = lib.tw_pack_f16(case["Wp"], G).to("cuda")
    At = _at(case["A"])
    C = H(lib.tw_gemm_f16(At, packed, out=torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")))
    check_f16(C, case["A"], case["Wp"], tw_terms(case["Wp"], G), f"tw {M}x{K}x{N} G={G}")
    Ct = H(lib.tw_gemm_f16_ex(At, packed, out_t=True,
                              out=torch.full((N, M), float("nan"), dtype=torch.float16, device="cuda")))
    assert np.array_equal(Ct.T.view(np.uint16), C.view(np.uint16))
    Cr = H(lib.tw_gemm_f16_ex(T(case["A"]), packed, a_rowmajor=True))
    assert np.array_equal(Cr.view(np.uint16), C.view(np.uint16))
    ex = wl.exact_int_tw_f16(np.random.default_rng(M + G), M, K, N, G, d)
    px = lib.tw_pack_f16(ex["Wp"], G).to("cuda")
    check_f16_exact(H(lib.tw_gemm_f16(_at(ex["A"]), px)), ex["A"], ex["Wp"], f"tw exact {M}x{K}x{N} G={G}")
    check_f16_exact(H(lib.tw_gemm_f16_ex(_at(ex["A"]), px, out_t=True)).T.copy(), ex["A"], ex["Wp"],
                    f"tw exact transposed out {M}x{K}x{N} G={G}")


@pytest.mark.parametrize("out", ["i32", "f16", "i8"])
@pytest.mark.parametrize("M,K,N,G,d", TW_LIMITS)
def test_tw_limits_i8(lib, gpu, M, K, N, G, d, out):
    rng = np.random.default_rng(M * 5 + K + G)
    case = wl.random_tw_i8(rng, M, K, N, G, d)
    scale = {"i32": None, "f16": case["scale"] * np.float32(20.0),
             "i8": rng.uniform(2e-4, 2e-3, size=N).astype(np.float32)}[out]
    bias = None if out == "i32" else rng.normal(0, 3.0, size=N).astype(np.float32)
    C = run_tw_i8(lib, case["A"], case["Wp"], G, scale, bias, out)
    ref = oracle.ref_gemm_i8_out(case["A"], case["Wp"], scale, bias, out)
    bad = np.flatnonzero(_bits(C) != _bits(ref))
    assert bad.size == 0, f"{bad.size} mismatches, first at {np.unravel_index(bad[0], C.shape)}"


# ---------------------------------------------------------------- transpose, determinism, errors
@pytest.mark.parametrize("M,K", [(8, 8), (136, 200), (4096, 768), (1000, 1024)])
def test_transpose_bit_exact(lib, gpu, M, K):
    A = wl.f16_normal(np.random.default_rng(M), (M, K))
    At = H(lib.ssg_transpose_f16(T(A)))
    assert np.array_equal(At.view(np.uint16), oracle.ref_transpose(A).view(np.uint16))


def test_determinism(lib, gpu):
    case = wl.random_24_f16(np.random.default_rng(12), 300, 1024, 512)
    a = run_w24_f16(lib, case["A"], case["Wp"])
    b = run_w24_f16(lib, case["A"], case["Wp"])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    c = wl.make_bert_base_fc1_tw()
    x = run_tw(lib, c["A"][:512], c["Wp"], 128)
    y = run_tw(lib, c["A"][:512], c["Wp"], 128)
    assert np.array_equal(x.view(np.uint16), y.view(np.uint16))


def test_w24_writes_every_output(lib, gpu):
    import torch
    case = wl.random_24_f16(np.random.default_rng(13), 77, 256, 192)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    out = torch.full((77, 192), float("nan"), dtype=torch.float16, device="cuda")
    C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), meta_t(meta), out=out))
    assert np.isfinite(C.astype(np.float32)).all()


# ---------------------------------------------------------------- largest operands
# The row-major GEMMs address A and W with 32-bit byte offsets and accept
# operands up to just under 4 GiB; the tile-wise kernels index At with 64-bit
# offsets.  Operands at those sizes are drawn on the GPU (integer values, so
# fp16 results are exact and compare bit for bit) and sampled output rows --
# the first and last 64 and 64 random ones -- are checked against the oracle.
def _sample_rows(M, seed):
    r = np.random.default_rng(seed).integers(0, M, 64)
    return np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), r]))


def _rows(t, rows):
    import torch
    return t.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()


def test_w24_largest_a(lib, gpu):
    import torch
    K, N = 1024, 64
    M = (1 << 32) // (2 * K) - 8  # A is 4 GiB - 16 KiB of fp16
    rows = _sample_rows(M, 41)
    w = wl.exact_int_24_f16(np.random.default_rng(41), 1, K, N)
    A = wl.device_int_matrix(torch, M, K, -3, 3, 41, torch.float16)
    vals, meta = lib.w24_pack_f16(w["Wp"])
    C = lib.w24_gemm_f16(A, T(vals), meta_t(meta))
    A_s, C_s = _rows(A, rows), _rows(C, rows)
    del A, C
    _, ref = oracle.ref_gemm_f16(A_s, w["Wp"])
    assert np.array_equal(C_s.view(np.uint16), ref.view(np.uint16))
    # int8 at the same row count (the limit check is the same for both kinds)
    c8 = wl.random_24_i8(np.random.default_rng(42), 1, K, N)
    A8 = wl.device_int_matrix(torch, M, K, -127, 127, 42, torch.int8)
    vals8, meta8 = lib.w24_pack_i8(c8["Wp"])
    C8 = lib.w24_gemm_i8(A8, T(vals8), meta_t(meta8), T(c8["scale"]))
    Cd = lib.dense_gemm_i8(A8, T(np.ascontiguousarray(c8["Wp"].T)), T(c8["scale"]))
    A8_s, C8_s, Cd_s = _rows(A8, rows), _rows(C8, rows), _rows(Cd, rows)
    ref8 = oracle.ref_gemm_i8(A8_s, c8["Wp"], c8["scale"])
    assert np.array_equal(C8_s.view(np.uint32), ref8.view(np.uint32))
    assert np.array_equal(Cd_s.view(np.uint32), ref8.view(np.uint32))


def test_tw_largest_at(lib, gpu):
    import torch
    K, N, G = 1024, 256, 128
    M = (1 << 31) // K + 16  # At holds more than 2^31 elements
    rows = _sample_rows(M, 43)
    c = wl.exact_int_tw_f16(np.random.default_rng(43), 1, K, N, G, [0.3, 0.7])
    At = wl.device_int_matrix(torch, K, M, -3, 3, 43, torch.float16)
    C = lib.tw_gemm_f16(At, lib.tw_pack_f16(c["Wp"], G).to("cuda"))
    idx = torch.from_numpy(rows).cuda()
    A_s = At.index_select(1, idx).t().contiguous().cpu().numpy()
    C_s = _rows(C, rows)
    del C
    _, ref = oracle.ref_gemm_f16(A_s, c["Wp"])
    assert np.array_equal(C_s.view(np.uint16), ref.view(np.uint16))
    # int8 tile-wise on the same At, as int8
    del At
    c8 = wl.random_tw_i8(np.random.default_rng(44), 1, K, N, G, [0.3, 0.7])
    At8 = wl.device_int_matrix(torch, K, M, -127, 127, 44, torch.int8)
    C8 = lib.tw_gemm_i8(At8, lib.tw_pack_i8(c8["Wp"], G).to("cuda"), T(c8["scale"]), None, out_type="f32")
    A8_s = At8.index_select(1, idx).t().contiguous().cpu().numpy()
    C8_s = _rows(C8, rows)
    ref8 = oracle.ref_gemm_i8_out(A8_s, c8["Wp"], c8["scale"], None, "f32")
    assert np.array_equal(C8_s.view(np.uint32), ref8.view(np.uint32))


def test_device_arch_is_gfx950(lib, gpu):
    assert lib.ssg_device_arch().startswith("gfx950")


def test_zero_tokens_is_noop(lib, gpu):
    import torch
    A = torch.empty((0, 128), dtype=torch.float16, device="cuda")
    vals, meta = lib.w24_pack_f16(np.zeros((128, 64), np.float16))
    C = lib.w24_gemm_f16(A, T(vals), meta_t(meta))
    assert C.shape == (0, 64)


# ---------------------------------------------------------------- randomised shapes
# A fixed, seeded draw of shapes inside each entry point's documented limits
# (2:4: K % 128 == 0 for int8 and % 64 for fp16, N % 64 == 0, any M; tile-wise:
# N % G == 0, G % 16 == 0, M % 8 (fp16) or % 16 (int8)), so tile-path choices,
# ragged token tails and K lengths not used elsewhere are all exercised.
def _random_shapes(seed, n, k_mult, m_mult, g_choices=None):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(r.integers(1, 3000)) // m_mult * m_mult or m_mult
        K = int(r.integers(1, 24)) * k_mult
        if g_choices is None:
            out.append((M, K, int(r.integers(1, 40)) * 64))
        else:
            G = int(r.choice(g_choices))
            out.append((M, K, int(r.integers(1, 24)) * G, G, float(r.uniform(0.05, 0.9))))
    return out


@pytest.mark.parametrize("M,K,N", _random_shapes(101, 6, 64, 1))
def test_w24_f16_random_shapes(lib, gpu, M, K, N):
    case = wl.random_24_f16(np.random.default_rng(M + K + N), M, K, N)
    check_f16(run_w24_f16(lib, case["A"], case["Wp"]), case["A"], case["Wp"], K // 2, f"2:4 f16 {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", _random_shapes(102, 6, 128, 1))
def test_w24_i8_random_shapes(lib, gpu, M, K, N):
    case = wl.random_24_i8(np.random.default_rng(M + K + N), M, K, N)
    C = run_w24_i8(lib, case["A"], case["Wp"], case["scale"])
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"]).view(np.uint32))
    Cd = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), T(case["scale"])))
    assert np.array_equal(Cd.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["W"], case["scale"]).view(np.uint32))


@pytest.mark.parametrize("M,K,N,G,d", _random_shapes(103, 6, 8, 8, [16, 32, 64, 128]))
def test_tw_random_shapes(lib, gpu, M, K, N, G, d):
    case = wl.random_tw_f16(np.random.default_rng(M + K + N), M, K, N, G, d)
    check_f16(run_tw(lib, case["A"], case["Wp"], G), case["A"], case["Wp"], tw_terms(case["Wp"], G),
              f"TW {M}x{K}x{N} G={G}")


@pytest.mark.parametrize("M,K,N,G,d", _random_shapes(104, 4, 16, 16, [16, 64, 128]))
def test_tw_i8_random_shapes(lib, gpu, M, K, N, G, d):
    rng = np.random.default_rng(M + K + N)
    case = wl.random_tw_i8(rng, M, K, N, G, d)
    C = run_tw_i8(lib, case["A"], case["Wp"], G, case["scale"], None, "f32")
    ref = oracle.ref_gemm_i8_out(case["A"], case["Wp"], case["scale"], None, "f32")
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- the element-wise comparison baseline
def test_elementwise_csr_baseline_matches_oracle(lib, gpu):
    """The pattern study's element-wise leg (torch's CSR sparse product in fp32,
    the slides' cuSparse stand-in) computes C = A . W_p: every fp16 x fp16
    product is exact in fp32, so it meets the fp32 summation bound."""
    import torch
    rng = np.random.default_rng(60)
    A = wl.f16_normal(rng, (256, 768))
    Wp = wl.prune_elementwise(wl.f16_normal(rng, (768, 384), 0.02), 0.37)
    S = torch.from_numpy(np.ascontiguousarray(Wp.T.astype(np.float32))).cuda().to_sparse_csr()
    At32 = torch.from_numpy(np.ascontiguousarray(A.T.astype(np.float32))).cuda()
    C = H(torch.sparse.mm(S, At32)).T
    C_ref = oracle.ref_gemm_f64(A, Wp)
    n = np.count_nonzero(Wp, axis=0).astype(np.float64)  # products per output column
    bound = 2.0 * n * 2.0 ** -24 * oracle.ref_abs_gemm(A, Wp) + 2.0 ** -126
    assert (np.abs(C.astype(np.float64) - C_ref) <= bound).all()
