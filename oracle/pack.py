"""Oracle packers (numpy).  Test infrastructure only.

2:4 format -- GPUSQ-ViT ("Boost Vision Transformer with GPU-Friendly Sparsity
and Quantization", abstract) prunes weights to the 2:4 fine-grained pattern:
at most two nonzeros in every four consecutive elements.  The pages fix no
storage format; the one used here (the reading adopted where they are silent):

* groups run along K inside one output column n: g covers k = 4g .. 4g+3;
* each group stores exactly two slots, positions i0 < i1 in 0..3.  The
  positions are the nonzero ones; a group with fewer than two nonzeros is
  filled with its lowest-index zero positions (two nonzeros -> those two; one
  nonzero p -> {p, lowest other}; none -> {0, 1}).  More than two -> error;
* ``vals[n, 2g + s]`` is the value at position i_s (a zero is stored as +0);
* ``meta[n, w]`` (uint32) holds 16 two-bit positions; slot j = 2g + s lives in
  word j // 16 at bits 2 * (j % 16).  Row stride is ceil(K / 32) words.

Tile-wise format -- "Accelerating Sparse DNN Models without Hardware-Support
via Tile-Wise Sparsity": tile t is the G-column slab [t*G, t*G+G) of W
spanning all of K (tile-wise pattern slide); offline preprocessing condenses
each tile into a dense block addressed through offset_k (kept rows, global
k) and offset_n (kept columns, tile-local) (run-time / preprocess slide).
The reading adopted here:

* a tile's kept columns are those with a nonzero in the tile, its kept rows
  the rows with a nonzero among the tile's columns, both ascending;
* the block V_t is stored [N_t x K_t] (K contiguous), each row padded with
  zeros to a multiple of ``TW_ROW_ALIGN_BYTES`` bytes (8 fp16 or 16 int8
  elements) so rows start 16-byte aligned; ``v_ptr`` counts padded elements;
* ``v_ptr``, ``k_ptr``, ``n_ptr`` are [T+1] prefix sums;
* ``tile_order`` lists tiles heaviest first (K_t * N_t descending, ties to the
  lower t): the longest-processing-time order used to schedule the grouped
  launch instead of one stream per tile.
"""

from __future__ import annotations

import numpy as np

TW_ROW_ALIGN_BYTES = 16


def _is_nonzero(W):
    """-0.0 counts as zero."""
    return np.asarray(W) != 0


def _canonical(vals):
    """Store every zero as +0."""
    vals = np.array(vals, copy=True)
    vals[vals == 0] = 0
    return vals


# ------------------------------------------------------------------ 2:4
def ref_prune24_mask(W):
    """Magnitude 2:4 mask, by rank: keep w[k] iff fewer than two entries of its
    group beat it, where w[j] beats w[k] if |w[j]| > |w[k]|, or the two are
    equal and j < k.  (The generator's pruner uses a sort; this is the rank
    definition, written independently, to cross-check it.)"""
    W = np.asarray(W)
    K, N = W.shape
    mag = np.abs(W.astype(np.float64)).reshape(K // 4, 4, N)
    beats = np.zeros(mag.shape, dtype=np.int64)
    for k in range(4):
        for j in range(4):
            if j == k:
                continue
            stronger = mag[:, j, :] > mag[:, k, :]
            if j < k:
                stronger |= mag[:, j, :] == mag[:, k, :]
            beats[:, k, :] += stronger
    return (beats < 2).reshape(K, N)


def ref_w24_positions(Wp):
    """Kept positions (i0, i1), each [K/4, N], following the canonical rule above."""
    Wp = np.asarray(Wp)
    K, N = Wp.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4")
    nz = _is_nonzero(Wp).reshape(K // 4, 4, N)
    count = nz.sum(axis=1)
    if (count > 2).any():
        g, n = np.argwhere(count > 2)[0]
        raise ValueError(f"group {g} of column {n} has {count[g, n]} nonzeros")
    # zero positions are ranked by index; the lowest (2 - count) of them fill
    zrank = np.cumsum(~nz, axis=1) - (~nz)
    keep = nz | (~nz & (zrank < (2 - count)[:, None, :]))
    assert (keep.sum(axis=1) == 2).all()
    pos = np.argsort(~keep, axis=1, kind="stable")[:, :2, :]  # kept positions, ascending
    return pos[:, 0, :], pos[:, 1, :]


def ref_w24_pack(Wp):
    """(vals [N, K/2], meta [N, ceil(K/32)] uint32) for a 2:4 weight W_p [K, N]."""
    Wp = np.asarray(Wp)
    K, N = Wp.shape
    i0, i1 = ref_w24_positions(Wp)
    groups = np.arange(K // 4)[:, None]
    cols = np.arange(N)[None, :]
    v0 = Wp[4 * groups + i0, cols]  # [K/4, N]
    v1 = Wp[4 * groups + i1, cols]
    vals = np.empty((N, K // 2), dtype=Wp.dtype)
    vals[:, 0::2] = v0.T
    vals[:, 1::2] = v1.T
    slots = np.empty((N, K // 2), dtype=np.uint64)
    slots[:, 0::2] = i0.T
    slots[:, 1::2] = i1.T
    words = -(-K // 32)
    meta = np.zeros((N, words), dtype=np.uint64)
    for j in range(K // 2):
        meta[:, j // 16] |= slots[:, j] << np.uint64(2 * (j % 16))
    return _canonical(vals), meta.astype(np.uint32)


def ref_w24_unpack(vals, meta, K, N):
    """Densify: W[4g + pos(slot), n] = vals[n, slot]; everything else +0."""
    vals = np.asarray(vals)
    meta = np.asarray(meta, dtype=np.uint32)
    W = np.zeros((K, N), dtype=vals.dtype)
    for j in range(K // 2):
        pos = (meta[:, j // 16] >> np.uint32(2 * (j % 16))) & np.uint32(3)
        k = 4 * (j // 2) + pos.astype(np.int64)
        W[k, np.arange(N)] = vals[:, j]
    return _canonical(W)


# ------------------------------------------------------------------ tile-wise
def ref_tw_structure(Wp, G):
    """Per tile: (kept rows as global k, kept columns tile-local), ascending."""
    Wp = np.asarray(Wp)
    K, N = Wp.shape
    out = []
    for c0 in range(0, N, G):
        nz = _is_nonzero(Wp[:, c0:min(N, c0 + G)])
        rows = np.flatnonzero(nz.any(axis=1))
        cols = np.flatnonzero(nz.any(axis=0))
        out.append((rows, cols))
    return out


def _round_up(x, a):
    return -(-x // a) * a


def ref_tw_pack(Wp, G):
    Wp = np.asarray(Wp)
    K, N = Wp.shape
    if G <= 0:
        raise ValueError("G must be positive")
    struct = ref_tw_structure(Wp, G)
    T = len(struct)
    v_ptr = np.zeros(T + 1, dtype=np.int64)
    k_ptr = np.zeros(T + 1, dtype=np.int64)
    n_ptr = np.zeros(T + 1, dtype=np.int64)
    blocks, oks, ons, work = [], [], [], []
    for t, (rows, cols) in enumerate(struct):
        kt, nt = len(rows), len(cols)
        ld = _round_up(kt, TW_ROW_ALIGN_BYTES // Wp.dtype.itemsize)
        blk = np.zeros((nt, ld), dtype=Wp.dtype)
        if kt and nt:
            blk[:, :kt] = Wp[np.ix_(rows, t * G + cols)].T
        blocks.append(blk.reshape(-1))
        oks.append(rows)
        ons.append(cols)
        v_ptr[t + 1] = v_ptr[t] + nt * ld
        k_ptr[t + 1] = k_ptr[t] + kt
        n_ptr[t + 1] = n_ptr[t] + nt
        work.append(kt * nt)
    tile_order = np.argsort(-np.asarray(work, dtype=np.int64), kind="stable")
    cat = (lambda xs, dt: np.concatenate(xs).astype(dt) if xs else np.zeros(0, dt))
    return dict(
        T=T,
        vals=_canonical(cat(blocks, Wp.dtype)),
        offset_k=cat(oks, np.int32),
        offset_n=cat(ons, np.int32),
        v_ptr=v_ptr.astype(np.int32),
        k_ptr=k_ptr.astype(np.int32),
        n_ptr=n_ptr.astype(np.int32),
        tile_order=tile_order.astype(np.int32),
    )


def ref_tw_unpack(packed, K, N, G):
    vals = packed["vals"]
    W = np.zeros((K, N), dtype=vals.dtype)
    vp, kp, np_ = packed["v_ptr"], packed["k_ptr"], packed["n_ptr"]
    for t in range(len(vp) - 1):
        kt, nt = int(kp[t + 1] - kp[t]), int(np_[t + 1] - np_[t])
        if kt == 0 or nt == 0:
            continue
        ld = (int(vp[t + 1]) - int(vp[t])) // nt
        blk = vals[vp[t]:vp[t + 1]].reshape(nt, ld)[:, :kt]
        rows = packed["offset_k"][kp[t]:kp[t + 1]]
        cols = packed["offset_n"][np_[t]:np_[t + 1]]
        W[np.ix_(rows, t * G + cols)] = blk.T
    return _canonical(W)
