"""Every GEMM and transpose entry point captured into a HIP graph and replayed.

The bench times the kernels as replayed graphs.  These tests check that each
launch captures (the kernels allocate nothing and record no memsets), that
every replay recomputes from the live input buffers (new inputs are copied in
place between replays), and that each replay equals an eager launch on the
same inputs bit for bit (the kernels are deterministic), with eager work and
synchronisations of the program's own between the replays.  The multi-stream
tile-wise schedule is captured too: its side streams fork from and join the
capturing stream.
"""

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _bits(t):
    import torch
    view = {torch.float16: torch.int16, torch.float32: torch.int32, torch.int32: torch.int32,
            torch.int8: torch.int8}[t.dtype]
    return t.view(view)


def _graph_replays(make_inputs, op):
    """make_inputs(seed) -> dict of device tensors (same shapes for every seed);
    op(inputs, out=None) -> output tensor."""
    import torch
    live = make_inputs(0)
    out = op(live)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up launch outside the capture
        op(live, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(live, out)
    for r in range(1, REPLAYS + 1):
        fresh = make_inputs(r)
        for k, v in fresh.items():
            live[k].copy_(v)
        expect = op(fresh)  # eager, on separate buffers
        torch.cuda.synchronize()
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(expect)), f"replay {r} differs from the eager launch"
    return out


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _f16(seed, shape):
    return wl.f16_normal(np.random.default_rng(seed), shape)


def _i8(seed, shape):
    return wl.i8_uniform(np.random.default_rng(seed), shape)


def test_graph_w24_f16(lib, gpu):
    M, K, N = 300, 512, 384
    W = wl.prune24_magnitude(wl.f16_normal(np.random.default_rng(100), (K, N), 0.02))
    vals, meta = lib.w24_pack_f16(W)
    v, m = _dev(vals), _dev(meta.view(np.int32))
    _graph_replays(lambda s: {"A": _dev(_f16(s, (M, K)))},
                   lambda x, out=None: lib.w24_gemm_f16(x["A"], v, m, out=out))


@pytest.mark.parametrize("K", [768, 2048])
def test_graph_w24_i8(lib, gpu, K):
    M, N = 300, 320
    rng = np.random.default_rng(101)
    W = wl.prune24_magnitude(wl.i8_weights(rng, (K, N)))
    vals, meta = lib.w24_pack_i8(W)
    v, m, sc = _dev(vals), _dev(meta.view(np.int32)), _dev(wl.f32_scales(rng, N))
    _graph_replays(lambda s: {"A": _dev(_i8(s, (M, K)))},
                   lambda x, out=None: lib.w24_gemm_i8(x["A"], v, m, sc, out=out))


@pytest.mark.parametrize("out_type", ["f16", "i8"])
def test_graph_w24_i8_out(lib, gpu, out_type):
    M, K, N = 200, 768, 256
    rng = np.random.default_rng(102)
    W = wl.prune24_magnitude(wl.i8_weights(rng, (K, N)))
    vals, meta = lib.w24_pack_i8(W)
    v, m = _dev(vals), _dev(meta.view(np.int32))
    sc, bi = _dev(wl.f32_scales(rng, N)), _dev(rng.normal(0, 1, N).astype(np.float32))
    _graph_replays(lambda s: {"A": _dev(_i8(s, (M, K)))},
                   lambda x, out=None: lib.w24_gemm_i8_out(x["A"], v, m, sc, bi, out_type=out_type, out=out))


def test_graph_dense_f16(lib, gpu):
    M, K, N = 200, 512, 384
    Wt = _dev(np.ascontiguousarray(wl.f16_normal(np.random.default_rng(103), (K, N), 0.02).T))
    _graph_replays(lambda s: {"A": _dev(_f16(s, (M, K)))},
                   lambda x, out=None: lib.dense_gemm_f16(x["A"], Wt, out=out))


def test_graph_dense_i8(lib, gpu):
    M, K, N = 200, 768, 320
    rng = np.random.default_rng(104)
    Wt = _dev(np.ascontiguousarray(wl.i8_weights(rng, (K, N)).T))
    sc = _dev(wl.f32_scales(rng, N))
    _graph_replays(lambda s: {"A": _dev(_i8(s, (M, K)))},
                   lambda x, out=None: lib.dense_gemm_i8(x["A"], Wt, sc, out=out))


def test_graph_transpose(lib, gpu):
    M, K = 296, 200
    _graph_replays(lambda s: {"A": _dev(_f16(s, (M, K)))},
                   lambda x, out=None: lib.ssg_transpose_f16(x["A"], out=out))


def _tw_weight(lib, K, N, G, seed):
    W = wl.prune_tilewise(wl.f16_normal(np.random.default_rng(seed), (K, N), 0.02), G, [0.3, 0.1, 0.6])
    return lib.tw_pack_f16(W, G).to("cuda")


def test_graph_tw_f16(lib, gpu):
    M, K, N, G = 256, 768, 384, 128
    p = _tw_weight(lib, K, N, G, 105)
    _graph_replays(lambda s: {"At": _dev(np.ascontiguousarray(_f16(s, (M, K)).T))},
                   lambda x, out=None: lib.tw_gemm_f16(x["At"], p, out=out))


@pytest.mark.parametrize("K", [768, 2048])  # narrow-tile kernels: 32-row stages; 64-row stages (K >= 2048)
@pytest.mark.parametrize("out_t", [False, True])
def test_graph_tw_f16_narrow(lib, gpu, K, out_t):
    M, N, G = 256, 384, 128
    W = wl.prune_tilewise(wl.f16_normal(np.random.default_rng(110), (K, N), 0.02), G, [0.2, 0.1, 0.25])
    p = lib.tw_pack_f16(W, G).to("cuda")
    assert p.narrow()
    _graph_replays(lambda s: {"At": _dev(np.ascontiguousarray(_f16(s, (M, K)).T))},
                   lambda x, out=None: lib.tw_gemm_f16_ex(x["At"], p, out_t=out_t, out=out))


@pytest.mark.parametrize("mode", ["out_t", "a_rowmajor"])
def test_graph_tw_f16_ex(lib, gpu, mode):
    M, K, N, G = 200, 512, 384, 128
    p = _tw_weight(lib, K, N, G, 106)
    if mode == "out_t":
        _graph_replays(lambda s: {"At": _dev(np.ascontiguousarray(_f16(s, (M, K)).T))},
                       lambda x, out=None: lib.tw_gemm_f16_ex(x["At"], p, out_t=True, out=out))
    else:
        _graph_replays(lambda s: {"A": _dev(_f16(s, (M, K)))},
                       lambda x, out=None: lib.tw_gemm_f16_ex(x["A"], p, a_rowmajor=True, out=out))


def test_graph_tw_f16_streams(lib, gpu):
    import torch
    M, K, N, G = 256, 512, 384, 128
    p = _tw_weight(lib, K, N, G, 107)
    streams = [torch.cuda.Stream() for _ in range(2)]
    _graph_replays(lambda s: {"At": _dev(np.ascontiguousarray(_f16(s, (M, K)).T))},
                   lambda x, out=None: lib.tw_gemm_f16_streams(x["At"], p, streams, out=out))


def test_graph_tw_i8(lib, gpu):
    M, K, N, G = 256, 768, 384, 128
    rng = np.random.default_rng(108)
    W = wl.prune_tilewise(wl.i8_weights(rng, (K, N)), G, [0.3, 0.1, 0.6])
    p = lib.tw_pack_i8(W, G).to("cuda")
    sc = _dev(wl.f32_scales(rng, N))
    _graph_replays(lambda s: {"At": _dev(np.ascontiguousarray(_i8(s, (M, K)).T))},
                   lambda x, out=None: lib.tw_gemm_i8(x["At"], p, sc, out_type="f16", out=out))


@pytest.mark.parametrize("kind", ["f16", "i8"])
def test_graph_splitk(lib, gpu, kind):
    """Split-K path (partial launch + reduce launch, workspace from torch's allocator
    inside the capture)."""
    M, K, N = 256, 4096, 256
    rng = np.random.default_rng(109)
    if kind == "f16":
        W = wl.prune24_magnitude(wl.f16_normal(rng, (K, N), 0.02))
        vals, meta = lib.w24_pack_f16(W)
        v, m = _dev(vals), _dev(meta.view(np.int32))
        _graph_replays(lambda s: {"A": _dev(_f16(s, (M, K)))},
                       lambda x, out=None: lib.w24_gemm_f16(x["A"], v, m, out=out, splits=8))
    else:
        W = wl.prune24_magnitude(wl.i8_weights(rng, (K, N)))
        vals, meta = lib.w24_pack_i8(W)
        v, m, sc = _dev(vals), _dev(meta.view(np.int32)), _dev(wl.f32_scales(rng, N))
        _graph_replays(lambda s: {"A": _dev(_i8(s, (M, K)))},
                       lambda x, out=None: lib.w24_gemm_i8(x["A"], v, m, sc, out=out, splits=4))
