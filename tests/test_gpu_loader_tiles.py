"""The tiles with loader waves and stage-blocked metadata, vs the oracle,
through the C ABI.

On the 128 x 128 tile that the fp16 GEMMs without enough 256 x 256 tiles
take (and the long-K int8 GEMMs with at most 256 such tiles), and on the
sparse fp16 64 x 128 tile, a second group of waves issues every
direct-to-LDS load, and the 2:4 kinds fetch their metadata in blocks of
several K stages (4 for fp16, 2 for int8), one block ahead, into a ring of
their own, where it is read at a swizzled position.  The cases cover the
edges of that arithmetic: a stage count that is not a multiple of the block
(a partial last block), fewer stages than one block, a single stage, K loops
that start at a rotated stage (every multi-tile sparse launch on these
tiles), ragged M and N, explicit K splits (each split starts its blocks at
its own first stage), one-hot weights (a metadata word read for the wrong
row or stage selects the wrong activation column), and every int8 output
kind.  The int8 2:4 tile runs stages of 256 k when K is a multiple of 256
(unsplit launches), of 128 k otherwise; both are covered, and the split
launches (128-k stages) are checked against the unsplit call.  Also here:
the fp16 2:4 256 x 256 tile, whose loads only its first four of eight
waves issue.  Bars as in the other parity tests: int8
bit-exact, fp16 within the strict per-element bound, and bit-exact on
exact-integer inputs.
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
    C_ref, _ = oracle.ref_gemm_f16(A, Wp)
    n_terms = Wp.shape[0] if dense else Wp.shape[0] // 2
    assert oracle.loose_err(C, C_ref) <= 1e-2, what
    assert oracle.strict_ok_f16(C, C_ref, oracle.ref_abs_gemm(A, Wp), n_terms), what


def _w24_f16(lib, A, Wp, splits=1):
    vals, meta = lib.w24_pack_f16(Wp)
    return H(lib.w24_gemm_f16(T(A), T(vals), T(meta.view(np.int32)), splits=splits))


# (M, K, N, tile): K stages of 64 fp16 k each
F16_CASES = [(2000, 832, 1088, (128, 128)),   # 16 x 9 tiles, 13 stages: last block partial
             (2000, 128, 1088, (128, 128)),   # 2 stages, less than one block
             (2000, 64, 1088, (128, 128)),    # a single stage
             (1300, 1024, 3008, (128, 128)),  # 11 x 24 tiles (264), 16 stages
             (1000, 704, 1088, (64, 128)),    # sparse 64 x 128 tile, 11 stages
             (1000, 192, 1088, (64, 128)),    # 3 stages
             (4000, 832, 3008, (256, 256)),   # 16 x 12 tiles of 256 x 256, half the waves load
             (4000, 64, 3008, (256, 256))]    # a single stage


@pytest.mark.parametrize("M,K,N,tile", F16_CASES)
def test_w24_f16_loader_tiles(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    case = wl.random_24_f16(np.random.default_rng(M + 3 * K), M, K, N)
    _check_f16(_w24_f16(lib, case["A"], case["Wp"]), case["A"], case["Wp"], f"w24 f16 {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,tile", F16_CASES[:2] + F16_CASES[4:5] + F16_CASES[6:7])
def test_w24_f16_loader_tiles_exact(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    case = wl.exact_int_24_f16(np.random.default_rng(K + N), M, K, N)
    _, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
    C = _w24_f16(lib, case["A"], case["Wp"])
    assert np.array_equal(C.view(np.uint16), C16.view(np.uint16))


@pytest.mark.parametrize("M,K,N,tile", [F16_CASES[0], F16_CASES[4], F16_CASES[6]])
def test_w24_f16_loader_tiles_one_hot(lib, gpu, M, K, N, tile):
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == tile
    case = wl.one_hot_24(np.random.default_rng(5), M, K, N)
    C = _w24_f16(lib, case["A"], case["Wp"])
    assert np.array_equal(C.view(np.uint16), case["A"][:, case["k_of_n"]].view(np.uint16))


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_w24_f16_loader_tile_splits(lib, gpu, splits):
    """16 stages over 2, 4 or 8 splits: blocks from each split's first stage."""
    M, K, N = 2000, 1024, 1088
    assert lib.tile_choice(lib.SSG_KIND_W24_F16, M, N, K) == (128, 128)
    case = wl.random_24_f16(np.random.default_rng(splits), M, K, N)
    C = _w24_f16(lib, case["A"], case["Wp"], splits=splits)
    _check_f16(C, case["A"], case["Wp"], f"w24 f16 {splits} splits")


def test_dense_f16_loader_tile(lib, gpu):
    M, K, N = 2000, 832, 1088
    assert lib.tile_choice(lib.SSG_KIND_DENSE_F16, M, N, K) == (128, 128)
    case = wl.random_24_f16(np.random.default_rng(41), M, K, N)
    C = H(lib.dense_gemm_f16(T(case["A"]), T(case["W"].T), splits=1))
    _check_f16(C, case["A"], case["W"], "dense f16 loader tile", dense=True)


# int8: the long-K rules (K > 1024) pick these tiles
I8_CASES = [(2000, 1152, 1088),   # 9 stages of 128 k: last metadata block of 2 partial
            (2000, 1280, 1088),   # 5 stages of 256 k
            (2000, 1536, 1088)]   # 6 stages of 256 k


@pytest.mark.parametrize("out", ["i32", "f32", "f16", "i8"])
@pytest.mark.parametrize("M,K,N", I8_CASES)
def test_w24_i8_loader_tiles_bit_exact(lib, gpu, out, M, K, N):
    assert lib.tile_choice(lib.SSG_KIND_W24_I8, M, N, K) == (128, 128)
    rng = np.random.default_rng(M + K + len(out))
    case = wl.random_24_i8(rng, M, K, N)
    bias = None if out == "i32" else rng.normal(0, 4, N).astype(np.float32)
    scale = None if out == "i32" else case["scale"]
    vals, meta = lib.w24_pack_i8(case["Wp"])
    C = H(lib.w24_gemm_i8_out(T(case["A"]), T(vals), T(meta.view(np.int32)), None if scale is None else T(scale),
                              None if bias is None else T(bias), out_type=out, splits=1))
    acc = oracle.ref_acc_i8(case["A"], case["Wp"])
    ref = acc if out == "i32" else oracle.ref_i8_epilogue(acc, scale, bias, out)
    assert np.array_equal(C.view(np.uint8), np.ascontiguousarray(ref).view(np.uint8))


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_w24_i8_loader_tile_splits(lib, gpu, splits):
    """16 stages over 2, 4 or 8 splits, bit-exact and equal to the unsplit call."""
    M, K, N = 2000, 2048, 1088
    assert lib.tile_choice(lib.SSG_KIND_W24_I8, M, N, K) == (128, 128)
    case = wl.random_24_i8(np.random.default_rng(60 + splits), M, K, N)
    vals, meta = lib.w24_pack_i8(case["Wp"])
    args = (T(case["A"]), T(vals), T(meta.view(np.int32)), T(case["scale"]))
    C = H(lib.w24_gemm_i8(*args, splits=splits))
    ref = oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"])
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(C.view(np.uint32), H(lib.w24_gemm_i8(*args, splits=1)).view(np.uint32))


def test_dense_i8_loader_tile(lib, gpu):
    M, K, N = 3000, 1152, 1088  # 24 x 9 = 216 tiles
    assert lib.tile_choice(lib.SSG_KIND_DENSE_I8, M, N, K) == (128, 128)
    case = wl.random_24_i8(np.random.default_rng(43), M, K, N)
    C = H(lib.dense_gemm_i8(T(case["A"]), T(case["W"].T), T(case["scale"]), splits=1))
    ref = oracle.ref_gemm_i8(case["A"], case["W"], case["scale"])
    assert np.array_equal(C.view(np.uint32), ref.view(np.uint32))
