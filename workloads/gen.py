"""Seeded input generators (numpy only).

Every workload is drawn from ``np.random.default_rng(seed)`` (PCG64) in a
fixed order, so both sides of a parity test see identical bytes.  Shapes and
distributions follow the five benchmark workloads:

* small -- 2:4 fp16, tiny: A[256x512] ~ U(-1,1), W[512x512] ~ N(0,0.02).
* vit_base_fc1 -- 2:4 int8, ViT-Base MLP fc1 (197 tokens x batch 64):
  A[12608x768] ~ U{-127..127}, W[768x3072] = clip(rint(N(0,32)), +-127),
  per-output-channel fp32 scale ~ U(1e-3, 1e-2).
* bert_base_fc1 -- tile-wise fp16, BERT-base FFN fc1 (seq 128 x batch 32):
  A[4096x768] ~ N(0,1), W[768x3072] ~ N(0,0.02), G = 128, 75 % global
  sparsity with uneven per-tile densities drawn from U(0.1,0.5).
* bert_large_ffn -- tile-wise fp16, BERT-large FFN (seq 384 x batch 16) at 90 %:
  fc1 A[6144x1024] W[1024x4096]; fc2 A[6144x4096] W[4096x1024]; G = 128.
* vit_large -- ViT-Large stack (256 tokens x batch 16 = 4096): per layer qkv
  (1024->3072), proj (1024->1024), fc1 (1024->4096), fc2 (4096->1024), 24
  layers, all 2:4, once in fp16 and once in int8.

The pruners are the synthetic stand-ins for the training-time pruning that
the pages describe (the pruned weight W_p is an *input* of the GEMM path).
"""

from __future__ import annotations

import numpy as np

F16 = np.float16
WORKLOAD_NAMES = ("small", "vit_base_fc1", "bert_base_fc1", "bert_large_ffn")


# ---------------------------------------------------------------- value draws
def f16_uniform(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, size=shape).astype(F16)


def f16_normal(rng, shape, std=1.0):
    return rng.normal(0.0, std, size=shape).astype(F16)


def i8_uniform(rng, shape):
    """Integers in [-127, 127] inclusive (never -128)."""
    return rng.integers(-127, 128, size=shape).astype(np.int8)


def i8_weights(rng, shape, std=32.0):
    """round-half-even(N(0, std)) clipped to [-127, 127]."""
    return np.clip(np.rint(rng.normal(0.0, std, size=shape)), -127, 127).astype(np.int8)


def f32_scales(rng, n, lo=1e-3, hi=1e-2):
    return rng.uniform(lo, hi, size=n).astype(np.float32)


def _plus_zero(w):
    """Replace -0.0 by +0.0 so pruned and underflowed entries are canonical."""
    w = np.array(w, copy=True)
    if w.dtype.kind == "f":
        w[w == 0] = 0
    return w


# ---------------------------------------------------------------- 2:4 pruner
def prune24_magnitude(W):
    """Keep the 2 largest |w| of each group of 4 consecutive K entries.

    W is [K x N]; groups run along K inside one output column.  Ties go to the
    lower k (stable sort on -|w|).  Magnitudes are taken on the stored dtype's
    values.  Pruned entries become +0.0 (or 0).
    """
    W = np.asarray(W)
    K, N = W.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4 for 2:4 pruning")
    mag = np.abs(W.astype(np.float64)).reshape(K // 4, 4, N)
    order = np.argsort(-mag, axis=1, kind="stable")
    keep = np.zeros_like(mag, dtype=bool)
    np.put_along_axis(keep, order[:, :2, :], True, axis=1)
    Wp = np.where(keep.reshape(K, N), W, np.zeros((), W.dtype)).astype(W.dtype)
    return _plus_zero(Wp)


# ---------------------------------------------------------------- TW pruner
def tile_shape(d, K, G):
    """(N_t, K_t) for a tile of density d: columns ~ G*sqrt(d), rows fill the rest."""
    if d <= 0.0:
        return 0, 0
    n_t = int(np.clip(np.rint(G * np.sqrt(d)), 1, G))
    k_t = int(np.clip(np.rint(d * K * G / n_t), 1, K))
    return n_t, k_t


def _top_indices(score, count):
    """Indices of the `count` largest scores, ties to the lower index, ascending."""
    order = np.argsort(-score, kind="stable")[:count]
    return np.sort(order)


def prune_tilewise(W, G, densities):
    """Tile-wise pruning of W [K x N] with G-column tiles.

    Tile t covers columns [t*G, (t+1)*G).  With density d_t it keeps N_t whole
    columns (largest L2 norm over all K) and then K_t whole rows (largest L2
    norm over the kept columns); everything else in the tile becomes +0.0.
    Norms are computed in float64 on the stored values.  d_t == 0 empties the
    tile.
    """
    W = np.asarray(W)
    K, N = W.shape
    T = -(-N // G)
    densities = np.broadcast_to(np.asarray(densities, dtype=np.float64), (T,))
    W64 = W.astype(np.float64)
    Wp = np.zeros_like(W)
    for t in range(T):
        c0, c1 = t * G, min(N, (t + 1) * G)
        g = c1 - c0
        n_t, k_t = tile_shape(float(densities[t]), K, g)
        if n_t == 0:
            continue
        blk = W64[:, c0:c1]
        cols = _top_indices(np.sqrt((blk * blk).sum(axis=0)), n_t)
        sub = blk[:, cols]
        rows = _top_indices(np.sqrt((sub * sub).sum(axis=1)), k_t)
        Wp[np.ix_(rows, c0 + cols)] = W[np.ix_(rows, c0 + cols)]
    return _plus_zero(Wp)


def prune_blockwise(W, b, density):
    """Block-wise (BW) pruning, the pattern the tile-wise slides compare against:
    W [K x N] is cut into b x b blocks; each block column keeps the
    round(density * K/b) blocks of largest L2 norm (ties to the lower block
    index, at least one), everything else becomes +0.  With G = b a BW weight is
    a tile-wise weight whose tiles keep whole b-row runs and every column."""
    W = np.asarray(W)
    K, N = W.shape
    if K % b or N % b:
        raise ValueError("K and N must be multiples of the block size")
    nkb = K // b
    keep = max(1, int(round(density * nkb)))
    W64 = W.astype(np.float64).reshape(nkb, b, N // b, b)
    norms = np.sqrt((W64 * W64).sum(axis=(1, 3)))  # [K/b, N/b]
    Wp = np.zeros_like(W)
    for jb in range(N // b):
        rows = _top_indices(norms[:, jb], keep)
        for kb in rows:
            Wp[kb * b:(kb + 1) * b, jb * b:(jb + 1) * b] = W[kb * b:(kb + 1) * b, jb * b:(jb + 1) * b]
    return _plus_zero(Wp)


def prune_elementwise(W, density):
    """Element-wise (EW, unstructured) magnitude pruning: every column keeps its
    round(density * K) entries of largest |w| (ties to the lower k)."""
    W = np.asarray(W)
    K, N = W.shape
    keep = max(1, int(round(density * K)))
    order = np.argsort(-np.abs(W.astype(np.float64)), axis=0, kind="stable")[:keep]
    Wp = np.zeros_like(W)
    cols = np.arange(N)[None, :]
    Wp[order, cols] = W[order, cols]
    return _plus_zero(Wp)


# ---------------------------------------------------------------- configs
def make_small_w24_f16(seed=0):
    rng = np.random.default_rng(seed)
    A = f16_uniform(rng, (256, 512))
    W = f16_normal(rng, (512, 512), 0.02)
    return dict(name="small_256x512x512", kind="w24_f16", M=256, K=512, N=512,
                A=A, W=W, Wp=prune24_magnitude(W))


def make_vit_base_fc1_i8(seed=0, M=64 * 197):
    rng = np.random.default_rng(seed)
    K, N = 768, 3072
    A = i8_uniform(rng, (M, K))
    W = i8_weights(rng, (K, N))
    scale = f32_scales(rng, N)
    return dict(name="vit_base_fc1", kind="w24_i8", M=M, K=K, N=N,
                A=A, W=W, Wp=prune24_magnitude(W), scale=scale)


def uneven_tile_densities(rng, T, target=0.25):
    """Uneven per-tile densities: u ~ U(0.1,0.5), rescaled to the global target."""
    u = rng.uniform(0.1, 0.5, size=T)
    return u * (target / u.mean())


def make_bert_base_fc1_tw(seed=0):
    rng = np.random.default_rng(seed)
    M, K, N, G = 32 * 128, 768, 3072, 128
    A = f16_normal(rng, (M, K))
    W = f16_normal(rng, (K, N), 0.02)
    d = uneven_tile_densities(rng, N // G)
    return dict(name="bert_base_fc1", kind="tw_f16", M=M, K=K, N=N, G=G,
                A=A, W=W, Wp=prune_tilewise(W, G, d), densities=d)


def make_bert_base_fc1_tw_i8(seed=0):
    """The BERT-base fc1 shape, tiles and densities with the integer path's
    data (int8 tile-wise): A int8 U{-127..127}, W round(N(0,32)) clipped,
    tile-wise pruned like the fp16 case, per-channel scales U(1e-3, 1e-2)."""
    rng = np.random.default_rng(seed)
    M, K, N, G = 32 * 128, 768, 3072, 128
    A = i8_uniform(rng, (M, K))
    W = i8_weights(rng, (K, N))
    d = uneven_tile_densities(rng, N // G)
    scale = f32_scales(rng, N)
    return dict(name="bert_base_fc1_i8", kind="tw_i8", M=M, K=K, N=N, G=G,
                A=A, W=W, Wp=prune_tilewise(W, G, d), densities=d, scale=scale)


def make_bert_large_ffn_tw(seed=0):
    rng = np.random.default_rng(seed)
    M, G = 16 * 384, 128
    A1 = f16_normal(rng, (M, 1024))
    W1 = f16_normal(rng, (1024, 4096), 0.02)
    A2 = f16_normal(rng, (M, 4096))
    W2 = f16_normal(rng, (4096, 1024), 0.02)
    fc1 = dict(name="bert_large_fc1", kind="tw_f16", M=M, K=1024, N=4096, G=G,
               A=A1, W=W1, Wp=prune_tilewise(W1, G, 0.1), densities=0.1)
    fc2 = dict(name="bert_large_fc2", kind="tw_f16", M=M, K=4096, N=1024, G=G,
               A=A2, W=W2, Wp=prune_tilewise(W2, G, 0.1), densities=0.1)
    return dict(name="bert_large_ffn", kind="tw_f16", fc1=fc1, fc2=fc2)


VIT_LARGE_M = 16 * 256
VIT_LARGE_GEMMS = (("qkv", 1024, 3072), ("proj", 1024, 1024),
              ("fc1", 1024, 4096), ("fc2", 4096, 1024))


def vit_large_layers(dtype="f16", seed=0, layers=24, M=VIT_LARGE_M):
    """Yield the 4*layers GEMMs of the ViT-Large stack, one dict at a time.

    fp16: A ~ N(0,1), W ~ N(0,0.02).  int8: the ViT-Base fc1 draws.  Every GEMM has
    its own A.  The fp16 and int8 stacks each start from default_rng(seed).
    """
    rng = np.random.default_rng(seed)
    for layer in range(layers):
        for gname, K, N in VIT_LARGE_GEMMS:
            if dtype == "f16":
                A = f16_normal(rng, (M, K))
                W = f16_normal(rng, (K, N), 0.02)
                yield dict(name=f"vit_large_l{layer}_{gname}", kind="w24_f16", M=M, K=K, N=N,
                           A=A, W=W, Wp=prune24_magnitude(W))
            elif dtype == "i8":
                A = i8_uniform(rng, (M, K))
                W = i8_weights(rng, (K, N))
                scale = f32_scales(rng, N)
                yield dict(name=f"vit_large_l{layer}_{gname}", kind="w24_i8", M=M, K=K, N=N,
                           A=A, W=W, Wp=prune24_magnitude(W), scale=scale)
            else:
                raise ValueError(dtype)


def make_workload(name, seed=0):
    return {"small": make_small_w24_f16, "vit_base_fc1": make_vit_base_fc1_i8,
            "bert_base_fc1": make_bert_base_fc1_tw, "bert_large_ffn": make_bert_large_ffn_tw}[name](seed)


# ---------------------------------------------------------------- small cases
def random_24_f16(rng, M, K, N, std_a=1.0, std_w=0.02):
    A = f16_normal(rng, (M, K), std_a)
    W = f16_normal(rng, (K, N), std_w)
    return dict(A=A, W=W, Wp=prune24_magnitude(W))


def random_tw_i8(rng, M, K, N, G, densities):
    A = i8_uniform(rng, (M, K))
    W = i8_weights(rng, (K, N))
    return dict(A=A, W=W, Wp=prune_tilewise(W, G, densities), scale=f32_scales(rng, N))


def random_24_i8(rng, M, K, N):
    A = i8_uniform(rng, (M, K))
    W = i8_weights(rng, (K, N))
    return dict(A=A, W=W, Wp=prune24_magnitude(W), scale=f32_scales(rng, N))


def random_tw_f16(rng, M, K, N, G, densities):
    A = f16_normal(rng, (M, K))
    W = f16_normal(rng, (K, N), 0.02)
    return dict(A=A, W=W, Wp=prune_tilewise(W, G, densities))


def exact_int_24_f16(rng, M, K, N):
    """A in {-3..3}, W in {-2..2} as fp16, pruned 2:4: every fp32 partial sum is exact."""
    A = rng.integers(-3, 4, size=(M, K)).astype(F16)
    W = rng.integers(-2, 3, size=(K, N)).astype(F16)
    return dict(A=A, W=W, Wp=prune24_magnitude(W))


def exact_int_tw_f16(rng, M, K, N, G, densities):
    A = rng.integers(-3, 4, size=(M, K)).astype(F16)
    W = rng.integers(-2, 3, size=(K, N)).astype(F16)
    return dict(A=A, W=W, Wp=prune_tilewise(W, G, densities))


def device_int_matrix(torch, rows, cols, lo, hi, seed, dtype):
    """Integer values in [lo, hi] drawn on the GPU by torch's seeded
    generator, as a rows x cols tensor of `dtype`: for operands of several
    GiB that would take too long to draw on the host and upload."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randint(lo, hi + 1, (rows, cols), generator=g, device="cuda", dtype=torch.int8)
    return x if dtype == torch.int8 else x.to(dtype)


def one_hot_24(rng, M, K, N, dtype=F16):
    """Each column n holds a single 1 at a random k(n); C[:, n] must equal A[:, k(n)]."""
    if dtype == np.int8:
        A = i8_uniform(rng, (M, K))
    else:
        A = f16_normal(rng, (M, K)).astype(dtype)
    kn = rng.integers(0, K, size=N)
    Wp = np.zeros((K, N), dtype=dtype)
    Wp[kn, np.arange(N)] = 1
    return dict(A=A, W=Wp, Wp=Wp, k_of_n=kn)


def one_hot_tw(rng, M, K, N, G, kept_cols_per_tile=3):
    """Tile-wise one-hot: in each tile a few columns hold a single 1 at a random k."""
    A = f16_normal(rng, (M, K))
    Wp = np.zeros((K, N), dtype=F16)
    kn = np.full(N, -1)
    for c0 in range(0, N, G):
        g = min(G, N - c0)
        cols = rng.choice(g, size=min(kept_cols_per_tile, g), replace=False)
        for c in cols:
            k = int(rng.integers(0, K))
            Wp[k, c0 + c] = 1
            kn[c0 + c] = k
    return dict(A=A, W=Wp, Wp=Wp, k_of_n=kn)
