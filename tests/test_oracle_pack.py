"""Pins for oracle/pack.py: exhaustive enumeration, closed-form metadata words,
round trips, structural invariants of the generated workloads, and planted
mistakes."""

import itertools

import numpy as np
import pytest

import oracle
import workloads as wl


# ---------------------------------------------------------------- 2:4 positions
def brute_positions(nonzero):
    """The canonical rule restated on one group of 4: the nonzero positions,
    topped up with the lowest zero positions, two in total, ascending."""
    nz = [i for i in range(4) if nonzero[i]]
    fill = [i for i in range(4) if not nonzero[i]]
    return tuple(sorted(nz + fill[:2 - len(nz)]))


ALL_PATTERNS = [p for p in itertools.product([0, 1], repeat=4) if sum(p) <= 2]


def test_positions_all_eleven_patterns():
    assert len(ALL_PATTERNS) == 11
    K = 4 * len(ALL_PATTERNS)
    W = np.zeros((K, 1), np.float16)
    for g, p in enumerate(ALL_PATTERNS):
        for i in range(4):
            if p[i]:
                W[4 * g + i, 0] = 1 + i
    i0, i1 = oracle.ref_w24_positions(W)
    for g, p in enumerate(ALL_PATTERNS):
        assert (int(i0[g, 0]), int(i1[g, 0])) == brute_positions(p)


def test_more_than_two_nonzeros_rejected():
    W = np.zeros((8, 2), np.int8)
    W[4:7, 1] = 1
    with pytest.raises(ValueError, match="group 1 of column 1"):
        oracle.ref_w24_pack(W)


def test_negative_zero_counts_as_zero():
    W = np.zeros((4, 1), np.float16)
    W[0, 0] = -0.0
    W[2, 0] = 0.5
    vals, meta = oracle.ref_w24_pack(W)
    assert int(meta[0, 0]) == (0 | 2 << 2)
    assert vals.view(np.uint16)[0, 0] == 0  # stored as +0


def test_meta_word_closed_form():
    # every group keeps positions (1, 3): each slot pair encodes 1 | 3 << 2 = 0xD
    K, N = 64, 3
    W = np.zeros((K, N), np.int8)
    W[1::4] = 5
    W[3::4] = -7
    vals, meta = oracle.ref_w24_pack(W)
    assert meta.shape == (N, 2) and (meta == 0xDDDDDDDD).all()
    assert (vals[:, 0::2] == 5).all() and (vals[:, 1::2] == -7).all()


def test_meta_ragged_words():
    # K = 36: 18 slots, 2 words per row, the second holds two slots
    K = 36
    W = np.zeros((K, 1), np.float16)
    W[K - 1, 0] = 1.0  # last group keeps (0, 3)
    _, meta = oracle.ref_w24_pack(W)
    assert meta.shape == (1, 2)
    assert int(meta[0, 0]) == 0x44444444  # positions (0, 1) -> 0 | 1 << 2 = 4
    assert int(meta[0, 1]) == (0 | 3 << 2)  # slots 16, 17 only


@pytest.mark.parametrize("dtype", ["f16", "i8"])
def test_w24_roundtrip_random(dtype):
    rng = np.random.default_rng(11)
    for K, N in [(128, 64), (768, 96), (36, 5)]:
        case = wl.random_24_f16(rng, 1, K, N) if dtype == "f16" else wl.random_24_i8(rng, 1, K, N)
        vals, meta = oracle.ref_w24_pack(case["Wp"])
        assert vals.shape == (N, K // 2) and meta.shape == (N, -(-K // 32))
        back = oracle.ref_w24_unpack(vals, meta, K, N)
        assert np.array_equal(back.view(np.uint8), case["Wp"].view(np.uint8))


def test_w24_pack_layout_closed_form():
    # Pack of a hand-built column against values read off the definition.
    W = np.zeros((8, 1), np.float16)
    W[2, 0], W[3, 0] = 3.0, -1.5   # group 0 keeps (2, 3)
    W[5, 0] = 0.25                 # group 1 keeps (0, 1) with 0.25 at position 1
    vals, meta = oracle.ref_w24_pack(W)
    assert vals.astype(np.float32).tolist() == [[3.0, -1.5, 0.0, 0.25]]
    assert int(meta[0, 0]) == (2 | 3 << 2) | ((0 | 1 << 2) << 4)


def test_prune_rank_definition_matches_generator():
    rng = np.random.default_rng(12)
    for W in (wl.i8_weights(rng, (96, 40)), wl.f16_normal(rng, (96, 40), 0.02),
              rng.integers(-1, 2, size=(64, 16)).astype(np.int8)):  # many ties
        mask = oracle.ref_prune24_mask(W)
        want = np.where(mask, W, np.zeros((), W.dtype))
        assert np.array_equal(want, wl.prune24_magnitude(W))
        assert (mask.reshape(-1, 4, W.shape[1]).sum(axis=1) == 2).all()


def test_generated_24_weights_have_at_most_two_per_group():
    for case in (wl.make_small_w24_f16(), wl.make_vit_base_fc1_i8()):
        Wp = case["Wp"]
        K, N = Wp.shape
        assert ((Wp != 0).reshape(K // 4, 4, N).sum(axis=1) <= 2).all()
        vals, meta = oracle.ref_w24_pack(Wp)
        assert np.array_equal(oracle.ref_w24_unpack(vals, meta, K, N), Wp)


# ---------------------------------------------------------------- tile-wise
def _check_tw_invariants(Wp, G, packed):
    K, N = Wp.shape
    T = packed["T"]
    assert T == -(-N // G)
    kp, np_, vp = packed["k_ptr"], packed["n_ptr"], packed["v_ptr"]
    assert kp[0] == np_[0] == vp[0] == 0
    for t in range(T):
        ks = packed["offset_k"][kp[t]:kp[t + 1]]
        ns = packed["offset_n"][np_[t]:np_[t + 1]]
        assert (np.diff(ks) > 0).all() and (np.diff(ns) > 0).all()
        if len(ks):
            assert 0 <= ks[0] and ks[-1] < K
        if len(ns):
            assert 0 <= ns[0] and ns[-1] < min(G, N - t * G)
        align = 16 // packed["vals"].dtype.itemsize  # rows padded to 16 bytes
        ld = align * -(-len(ks) // align)
        assert vp[t + 1] - vp[t] == len(ns) * ld
        # zero outside kept rows x kept columns
        win = Wp[:, t * G:(t + 1) * G].copy()
        win[np.ix_(ks, ns)] = 0
        assert not win.any()
    order = packed["tile_order"]
    assert sorted(order.tolist()) == list(range(T))
    work = np.diff(kp) * np.diff(np_)
    assert (np.diff(work[order]) <= 0).all()


def test_tw_small_roundtrip_and_invariants():
    rng = np.random.default_rng(13)
    for (K, N, G, d) in [(64, 48, 16, [0.3, 1.0, 0.0]), (100, 40, 16, 0.5), (33, 10, 4, 0.4)]:
        case = wl.random_tw_f16(rng, 1, K, N, G, d)
        packed = oracle.ref_tw_pack(case["Wp"], G)
        _check_tw_invariants(case["Wp"], G, packed)
        assert np.array_equal(oracle.ref_tw_unpack(packed, K, N, G).view(np.uint16),
                              case["Wp"].view(np.uint16))


def test_tw_full_density_tile_is_dense():
    rng = np.random.default_rng(14)
    W = wl.f16_normal(rng, (24, 16), 1.0)
    packed = oracle.ref_tw_pack(W, 16)
    assert packed["T"] == 1 and list(packed["offset_k"]) == list(range(24))
    blk = packed["vals"].reshape(16, 24)
    assert np.array_equal(blk, W.T)


def test_tw_bert_structure():
    c3 = wl.make_bert_base_fc1_tw()
    p3 = oracle.ref_tw_pack(c3["Wp"], 128)
    _check_tw_invariants(c3["Wp"], 128, p3)
    kt, nt = np.diff(p3["k_ptr"]), np.diff(p3["n_ptr"])
    for t in range(24):
        assert (nt[t], kt[t]) == wl.tile_shape(c3["densities"][t], 768, 128)
    density = (kt * nt).sum() / (768 * 3072)
    assert abs(density - 0.25) < 0.005
    c4 = wl.make_bert_large_ffn_tw()
    for sub, K, T in ((c4["fc1"], 1024, 32), (c4["fc2"], 4096, 8)):
        p = oracle.ref_tw_pack(sub["Wp"], 128)
        _check_tw_invariants(sub["Wp"], 128, p)
        assert p["T"] == T
        assert (np.diff(p["n_ptr"]) == 40).all()
        assert (np.diff(p["k_ptr"]) == (328 if K == 1024 else 1311)).all()


# ---------------------------------------------------------------- planted mistakes
def test_roundtrip_catches_wrong_meta_shift():
    rng = np.random.default_rng(15)
    case = wl.random_24_f16(rng, 1, 64, 8)
    vals, meta = oracle.ref_w24_pack(case["Wp"])
    bad = ((meta << np.uint32(2)) | (meta >> np.uint32(30))).astype(np.uint32)  # slot off by one
    assert not np.array_equal(oracle.ref_w24_unpack(vals, bad, 64, 8), case["Wp"])


def test_enumeration_catches_wrong_fill_rule():
    def highest_fill(nonzero):
        nz = [i for i in range(4) if nonzero[i]]
        fill = [i for i in reversed(range(4)) if not nonzero[i]]
        return tuple(sorted(nz + fill[:2 - len(nz)]))
    assert any(highest_fill(p) != brute_positions(p) for p in ALL_PATTERNS)
