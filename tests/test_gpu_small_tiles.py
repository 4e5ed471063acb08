"""The small tiles (64 x 64, 64 x 128 and one-wave 32 x 32) that GEMMs with
few output tiles take, vs the oracle, through the C ABI.

Each case first asserts, through the library's host-side tile query, that
its shape reaches the tile it is meant to cover, so that a change of the
tile rules cannot leave a path untested.  Covered: the fp16 2:4 64 x 64 tile,
where two waves load each meta chunk of a stage; 64 x 128 fp16 tiles; 32 x 32
tiles; ragged
token counts (M not a multiple of 64); every int8 output kind bit-exact; the
dense kinds; and split K on 64 x 64 tiles.  Bars as in the other parity
tests: int8 bit-exact, fp16 within the strict per-element bound and
bit-exact on exact-integer inputs.
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
    sums: K for the dense kinds, K/2 kept slots for the 2:4 kinds."""
    C_ref, _ = oracle.ref_gemm_f16(A, Wp)
    n_terms = Wp.shape[0] if dense else Wp.shape[0] // 2
    assert oracle.loose_err(C, C_ref) <= 1e-2, what
    assert oracle.strict_ok_f16(C, C_ref, oracle.ref_abs_gemm(A, Wp), n_terms), what


# (M, K, N, tile the fp16 kinds take)
F16_CASES = [(600, 512, 1024, (64, 64)),    # 10 x 16 tiles, last tile row 24 rows deep
             (1000, 256, 2048, (64, 128)),  # 64 x 64 tiles would number 512
             (64, 4096, 128, (64, 64)),     # one tile row, 64 K stages
             (200, 512, 256, (32, 32)),     # 7 x 8 tiles, last tile row 8 rows deep
             (1, 128, 64, (32, 32))]        # a single token


@pytest.mark.parametrize("M,K,N,tile", F16_CASES)
def test_w24_f16_small_tiles(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    case = wl.random_24_f16(np.random.default_rng(M + K), M, K, N)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), T(meta.view(np.int32)), splits=1))
    _check_f16(C, case["A"], case["Wp"], f"w24 f16 {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,tile", F16_CASES[:2])
def test_w24_f16_small_tiles_exact(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    case = wl.exact_int_24_f16(np.random.default_rng(7 + M), M, K, N)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), T(meta.view(np.int32)), splits=1))
    _, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
    assert np.array_equal(C.view(np.uint16), C16.view(np.uint16))


def test_w24_f16_64x64_one_hot(lib, gpu):
    """Each output column copies one activation column: a meta chunk loaded for
    the wrong channel rows, or missing from the stage, selects the wrong k."""
    for M, K, N, tile in ((600, 512, 1024, (64, 64)), (96, 1024, 192, (32, 32))):
        assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
        case = wl.one_hot_24(np.random.default_rng(11), M, K, N)
        vals, meta = lib.w24_pack_f16(case["Wp"])
        C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), T(meta.view(np.int32)), splits=1))
        assert np.array_equal(C.view(np.uint16), case["A"][:, case["k_of_n"]].view(np.uint16)), tile


@pytest.mark.parametrize("M,K,N,tile", F16_CASES[:2])
def test_dense_f16_small_tiles(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_DENSE_F16, M, N, K) == tile
    case = wl.random_24_f16(np.random.default_rng(3 + M), M, K, N)
    C = H(lib.dense_gemm_f16(T(case["A"]), T(case["W"].T), splits=1))
    _check_f16(C, case["A"], case["W"], f"dense f16 {M}x{K}x{N}", dense=True)


@pytest.mark.parametrize("out", ["i32", "f32", "f16", "i8"])
@pytest.mark.parametrize("M,K,N,tile", [(200, 1024, 320, (32, 32)), (1000, 256, 2048, (64, 64))])
def test_w24_i8_small_tiles_bit_exact(lib, gpu, out, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_I8, M, N, K) == tile
    rng = np.random.default_rng(M + N)
    case = wl.random_24_i8(rng, M, K, N)
    bias = None if out == "i32" else rng.normal(0, 4, N).astype(np.float32)
    scale = None if out == "i32" else case["scale"]
    vals, meta = lib.w24_pack_i8(case["Wp"])
    C = H(lib.w24_gemm_i8_out(T(case["A"]), T(vals), T(meta.view(np.int32)), None if scale is None else T(scale),
                              None if bias is None else T(bias), out_type=out, splits=1))
    acc = oracle.ref_acc_i8(case["A"], case["Wp"])
    ref = acc if out == "i32" else oracle.ref_i8_epilogue(acc, scale, bias, out)
    assert np.array_equal(C.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


@pytest.mark.parametrize("out", ["i32", "f32", "i8"])
@pytest.mark.parametrize("M,K,N,tile", [(136, 768, 448, (32, 32)), (600, 768, 1024, (64, 64))])
def test_dense_i8_small_tiles_bit_exact(lib, gpu, out, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_DENSE_I8, M, N, K) == tile
    rng = np.random.default_rng(17)
    case = wl.random_24_i8(rng, M, K, N)
    scale = None if out == "i32" else case["scale"]
    C = H(lib.dense_gemm_i8_out(T(case["A"]), T(case["W"].T), None if scale is None else T(scale), None,
                                out_type=out, splits=1))
    acc = oracle.ref_acc_i8(case["A"], case["W"])
    ref = acc if out == "i32" else oracle.ref_i8_epilogue(acc, scale, None, out)
    assert np.array_equal(C.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


def test_i8_short_k_192_tiles(lib, gpu):
    """int8 with K <= 1024 keeps 64 x 64 tiles up to 192 tiles of 128 x 128."""
    M, K, N = 1528, 256, 2048  # 12 x 16 tiles of 128 x 128, last row of 64-row tiles ragged
    rng = np.random.default_rng(31)
    case = wl.random_24_i8(rng, M, K, N)
    for kind in (lib.SSG_KIND_W24_I8, lib.SSG_KIND_DENSE_I8):
        assert lib.tile_choice(kind, M, N, K) == (64, 64)
    vals, meta = lib.w24_pack_i8(case["Wp"])
    C = H(lib.w24_gemm_i8(T(case["A"]), T(vals), T(meta.view(np.int32)), T(case["scale"])))
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"]).view(np.uint32))
    C = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), None))
    assert np.array_equal(C, oracle.ref_acc_i8(case["A"], case["W"]))


def test_split_k_on_64x64_tiles(lib, gpu):
    """Long K, few 64 x 64 tiles: the library splits on its own; int8 stays
    bit-exact (and equal to the unsplit call) and fp16 within the bound."""
    M, K, N = 72, 8192, 128
    assert lib.tile_choice(lib.SSG_KIND_W24_I8, M, N, K) == (64, 64)
    p8 = lib.splitk_suggest(lib.SSG_KIND_W24_I8, M, N, K)
    assert p8 > 1
    case = wl.random_24_i8(np.random.default_rng(23), M, K, N)
    vals, meta = lib.w24_pack_i8(case["Wp"])
    args = (T(case["A"]), T(vals), T(meta.view(np.int32)), T(case["scale"]))
    C = H(lib.w24_gemm_i8(*args))
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"]).view(np.uint32))
    assert np.array_equal(C.view(np.uint32), H(lib.w24_gemm_i8(*args, splits=1)).view(np.uint32))

    K16 = 4096
    assert lib.splitk_suggest(lib.SSG_KIND_W24_F16, M, N, K16) > 1
    case = wl.random_24_f16(np.random.default_rng(29), M, K16, N)
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), T(meta.view(np.int32))))
    _check_f16(C, case["A"], case["Wp"], "w24 f16 split on 64x64")


# Shapes on both sides of each tile-rule boundary: (kind, M, K, N, tile).
F16_BOUNDARY = [(512, 128, 1024, (32, 32)),      # 512 tiles of 32 x 32
                (520, 128, 1024, (64, 64)),      # 544
                (512, 4032, 1024, (32, 32)),     # 63 K stages
                (512, 4096, 1024, (64, 64)),     # 64 stages: 64 x 64 (unsplit; the default call splits)
                (1024, 128, 1024, (64, 64)),     # 256 tiles of 64 x 64
                (1032, 128, 1024, (64, 128)),    # 272 would be too many
                (1024, 128, 2048, (64, 128)),    # 128 tiles of 128 x 128
                (1032, 128, 2048, (128, 128))]   # 144: not few any more
I8_BOUNDARY = [(512, 128, 1024, (32, 32)),       # 512 tiles of 32 x 32
               (520, 128, 1024, (64, 64)),       # 544
               (128, 8064, 256, (32, 32)),       # 63 K stages
               (128, 8192, 256, (64, 64)),       # 64
               (1536, 256, 2048, (64, 64)),      # short K: 192 tiles of 128 x 128
               (1544, 256, 2048, (128, 128)),    # 208
               (1024, 1152, 2048, (64, 64)),     # long K: 128
               (1032, 1152, 2048, (128, 128))]   # 144


# The tile query describes the unsplit launch, so these cases call the GEMMs
# with splits=1: the asserted tile is the one that runs.
@pytest.mark.parametrize("M,K,N,tile", F16_BOUNDARY)
def test_f16_tile_rule_boundaries(lib, gpu, M, K, N, tile):
    case = wl.random_24_f16(np.random.default_rng(M * 7 + N), M, K, N)
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    assert lib.tile_choice(lib.SSG_KIND_DENSE_F16, M, N, K) == tile
    vals, meta = lib.w24_pack_f16(case["Wp"])
    C = H(lib.w24_gemm_f16(T(case["A"]), T(vals), T(meta.view(np.int32)), splits=1))
    _check_f16(C, case["A"], case["Wp"], f"w24 f16 {M}x{K}x{N}")
    C = H(lib.dense_gemm_f16(T(case["A"]), T(case["W"].T), splits=1))
    _check_f16(C, case["A"], case["W"], f"dense f16 {M}x{K}x{N}", dense=True)


@pytest.mark.parametrize("M,K,N,tile", I8_BOUNDARY)
def test_i8_tile_rule_boundaries(lib, gpu, M, K, N, tile):
    case = wl.random_24_i8(np.random.default_rng(M * 5 + K), M, K, N)
    assert lib.tile_choice(lib.SSG_KIND_W24_I8, M, N, K) == tile
    assert lib.tile_choice(lib.SSG_KIND_DENSE_I8, M, N, K) == tile
    vals, meta = lib.w24_pack_i8(case["Wp"])
    C = H(lib.w24_gemm_i8(T(case["A"]), T(vals), T(meta.view(np.int32)), T(case["scale"]), splits=1))
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"]).view(np.uint32))
    C = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), T(case["scale"]), splits=1))
    assert np.array_equal(C.view(np.uint32), oracle.ref_gemm_i8(case["A"], case["W"], case["scale"]).view(np.uint32))
