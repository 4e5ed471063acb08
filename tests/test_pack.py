"""Host packers of libssg vs the oracle's packers: byte-identical output,
round trips, and the documented error codes (CPU only)."""

import ctypes as ct

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import workloads as wl


def assert_same_bytes(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape and a.dtype.itemsize == b.dtype.itemsize
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def adversarial_24(rng, K, N, dtype):
    """Groups with 0, 1 or 2 nonzeros at every position, ties, -0.0."""
    W = np.zeros((K, N), dtype)
    for g in range(K // 4):
        for n in range(N):
            k = rng.integers(0, 3)
            pos = rng.choice(4, size=k, replace=False)
            for p in pos:
                W[4 * g + p, n] = rng.choice([1, -1, 2, 3]) if dtype == np.int8 else rng.choice([1.0, -0.5, 2.0])
    if dtype == np.float16:
        W[(W == 0) & (rng.random(W.shape) < 0.3)] = -0.0
    return W


@pytest.mark.parametrize("dtype", [np.float16, np.int8])
@pytest.mark.parametrize("K,N", [(4, 1), (36, 5), (128, 64), (768, 96)])
def test_w24_pack_matches_oracle(lib, dtype, K, N):
    rng = np.random.default_rng(K * N)
    for W in (adversarial_24(rng, K, N, dtype),
              (wl.random_24_f16(rng, 1, K, N)["Wp"] if dtype == np.float16 else wl.random_24_i8(rng, 1, K, N)["Wp"])):
        pack = lib.w24_pack_f16 if dtype == np.float16 else lib.w24_pack_i8
        unpack = lib.w24_unpack_f16 if dtype == np.float16 else lib.w24_unpack_i8
        vals, meta = pack(W)
        rv, rm = oracle.ref_w24_pack(W)
        assert_same_bytes(vals, rv)
        assert_same_bytes(meta, rm)
        back = unpack(vals, meta, K, N)
        assert_same_bytes(back, oracle.ref_w24_unpack(rv, rm, K, N))
        assert np.array_equal(back.astype(np.float64), W.astype(np.float64))  # value round trip


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 24), st.integers(1, 9), st.integers(0, 2**32 - 1))
def test_w24_pack_property(lib, groups, N, seed):
    rng = np.random.default_rng(seed)
    W = adversarial_24(rng, 4 * groups, N, np.float16)
    vals, meta = lib.w24_pack_f16(W)
    rv, rm = oracle.ref_w24_pack(W)
    assert_same_bytes(vals, rv)
    assert_same_bytes(meta, rm)


def test_w24_pack_full_configs(lib):
    for c in (wl.make_small_w24_f16(), wl.make_vit_base_fc1_i8()):
        pack = lib.w24_pack_f16 if c["Wp"].dtype == np.float16 else lib.w24_pack_i8
        vals, meta = pack(c["Wp"])
        rv, rm = oracle.ref_w24_pack(c["Wp"])
        assert_same_bytes(vals, rv)
        assert_same_bytes(meta, rm)


def test_w24_pack_errors(lib):
    W = np.zeros((8, 3), np.float16)
    W[4:7, 2] = 1.0
    with pytest.raises(lib.SsgError, match="SSG_ENOT24.*group 1 of column 2"):
        lib.w24_pack_f16(W)
    with pytest.raises(lib.SsgError, match="SSG_EINVAL.*multiple of 4"):
        lib.w24_pack_i8(np.zeros((6, 2), np.int8))


def test_w24_unpack_rejects_bad_positions(lib):
    vals = np.zeros((1, 2), np.float16)
    meta = np.array([[3 | (1 << 2)]], np.uint32)  # positions (3, 1): not ascending
    with pytest.raises(lib.SsgError, match="not ascending"):
        lib.w24_unpack_f16(vals, meta, 4, 1)


def _tw_equal(p, ref):
    assert p.T == ref["T"]
    for k in ("vals", "offset_k", "offset_n", "v_ptr", "k_ptr", "n_ptr", "tile_order"):
        assert_same_bytes(getattr(p, k), ref[k])


@pytest.mark.parametrize("K,N,G,d", [(64, 48, 16, [0.3, 1.0, 0.0]), (100, 40, 16, 0.5), (33, 10, 4, 0.4),
                                     (768, 384, 128, [0.1, 0.4, 0.25])])
def test_tw_pack_matches_oracle(lib, K, N, G, d):
    case = wl.random_tw_f16(np.random.default_rng(K + N), 1, K, N, G, d)
    W = case["Wp"].copy()
    W[(W == 0) & (np.random.default_rng(1).random(W.shape) < 0.2)] = -0.0
    p = lib.tw_pack_f16(W, G)
    _tw_equal(p, oracle.ref_tw_pack(W, G))
    assert np.array_equal(lib.tw_unpack_f16(p).astype(np.float64), W.astype(np.float64))


@pytest.mark.parametrize("K,N,G,d", [(64, 48, 16, [0.3, 1.0, 0.0]), (100, 40, 16, 0.5), (33, 10, 4, 0.4),
                                     (768, 384, 128, [0.1, 0.4, 0.25])])
def test_tw_pack_i8_matches_oracle(lib, K, N, G, d):
    case = wl.random_tw_i8(np.random.default_rng(K + 2 * N), 1, K, N, G, d)
    p = lib.tw_pack_i8(case["Wp"], G)
    assert p.vals.dtype == np.int8
    ref = oracle.ref_tw_pack(case["Wp"], G)
    _tw_equal(p, ref)
    # int8 rows are padded to 16 elements (16 bytes)
    for t in range(p.T):
        kt, nt = p.k_ptr[t + 1] - p.k_ptr[t], p.n_ptr[t + 1] - p.n_ptr[t]
        assert p.v_ptr[t + 1] - p.v_ptr[t] == nt * (-(-kt // 16) * 16)
    assert np.array_equal(lib.tw_unpack_i8(p), case["Wp"])


def test_tw_pack_i8_workload(lib):
    c = wl.make_bert_base_fc1_tw_i8()
    _tw_equal(lib.tw_pack_i8(c["Wp"], 128), oracle.ref_tw_pack(c["Wp"], 128))


def test_tw_pack_full_configs(lib):
    c3 = wl.make_bert_base_fc1_tw()
    _tw_equal(lib.tw_pack_f16(c3["Wp"], 128), oracle.ref_tw_pack(c3["Wp"], 128))
    c4 = wl.make_bert_large_ffn_tw()
    for sub in (c4["fc1"], c4["fc2"]):
        _tw_equal(lib.tw_pack_f16(sub["Wp"], 128), oracle.ref_tw_pack(sub["Wp"], 128))


def test_tw_query_and_enospc(lib):
    case = wl.random_tw_f16(np.random.default_rng(2), 1, 64, 32, 16, 0.5)
    q = lib.tw_pack_query(case["Wp"], 16)
    ref = oracle.ref_tw_pack(case["Wp"], 16)
    assert q["T"] == 2 and q["sum_kt"] == len(ref["offset_k"]) and q["vals_elems"] == len(ref["vals"])
    raw = lib.load()
    cap = lib._lib.TwSizes(q["T"], q["sum_kt"], q["sum_nt"], q["vals_elems"] - 1)
    bufs = [np.empty(max(1, n), dt) for n, dt in ((q["vals_elems"], np.uint16), (q["sum_kt"], np.int32),
                                                  (q["sum_nt"], np.int32), (3, np.int32), (3, np.int32),
                                                  (3, np.int32), (2, np.int32))]
    W = np.ascontiguousarray(case["Wp"])
    rc = raw.tw_pack_f16(W.ctypes.data_as(ct.c_void_p), 64, 32, 16, ct.byref(cap),
                         *[b.ctypes.data_as(ct.c_void_p) for b in bufs])
    assert rc == 3 and "capacity" in raw.ssg_last_error().decode()


def test_tw_unpack_rejects_inconsistent_pointers(lib):
    case = wl.random_tw_f16(np.random.default_rng(3), 1, 32, 32, 16, 0.5)
    p = lib.tw_pack_f16(case["Wp"], 16)
    p.v_ptr = p.v_ptr.copy()
    p.v_ptr[1] += 1
    with pytest.raises(lib.SsgError, match="inconsistent"):
        lib.tw_unpack_f16(p)


def test_tw_unpack_rejects_bad_prefix_sums_and_lengths(lib):
    import copy
    case = wl.random_tw_f16(np.random.default_rng(4), 1, 32, 32, 16, 0.5)
    p0 = lib.tw_pack_f16(case["Wp"], 16)
    p = copy.copy(p0)
    p.k_ptr = p0.k_ptr - 1  # every tile keeps its size, but the sums start at -1
    with pytest.raises(lib.SsgError, match="start at 0"):
        lib.tw_unpack_f16(p)
    p = copy.copy(p0)
    p.n_ptr = p0.n_ptr[:-1]
    with pytest.raises(ValueError, match="T\\+1"):
        lib.tw_unpack_f16(p)
    p = copy.copy(p0)
    p.offset_k = p0.offset_k[:-1]
    with pytest.raises(ValueError, match="shorter"):
        lib.tw_unpack_f16(p)
    # raw C ABI: a null offset array with a nonzero length is refused
    raw = lib.load()
    import ctypes as ct
    W = np.empty((32, 32), np.float16)
    arrs = [np.ascontiguousarray(a) for a in (p0.vals, p0.offset_k, p0.offset_n, p0.v_ptr, p0.k_ptr, p0.n_ptr)]
    ptrs = [a.ctypes.data_as(ct.c_void_p) for a in arrs]
    ptrs[1] = None
    rc = raw.tw_unpack_f16(*ptrs, 32, 32, 16, W.ctypes.data_as(ct.c_void_p))
    assert rc == 1 and "null array" in raw.ssg_last_error().decode()


@pytest.mark.parametrize("G,d,narrow", [(128, [0.1, 0.25], True), (128, [0.1, 0.26], False),
                                        (64, [1.0, 0.5], True), (32, 1.0, True), (256, [0.05, 0.06], True),
                                        (128, [0.0, 0.0], True)])
def test_tw_pack_reports_widest_tile(lib, G, d, narrow):
    """The host pack records the most kept columns of any tile (what the binding's
    SSG_TW_NARROW choice rests on): max over tiles of n_ptr[t+1] - n_ptr[t]."""
    case = wl.random_tw_f16(np.random.default_rng(G), 16, 256, 2 * G, G, d)
    packed = lib.tw_pack_f16(case["Wp"], G)
    ref = oracle.ref_tw_pack(case["Wp"], G)
    assert packed.max_nt == int(np.diff(ref["n_ptr"]).max())
    assert packed.narrow() == narrow == (packed.max_nt <= 64)
    # a hand-built pack with no column count known takes the general path
    assert not lib.TwPacked(packed.K, packed.N, packed.G, packed.T, *packed.arrays().values()).narrow()
