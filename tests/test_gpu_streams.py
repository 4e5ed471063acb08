"""Entry points running at the same time on several streams.

The library keeps no device state between calls, so GEMMs launched
concurrently on different streams must give exactly the results they give
when run one after another on one stream.  Each stream's operands and
output are its own; everything is bit-compared (the kernels are
deterministic).
"""

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.float16 else torch.int32)


def test_concurrent_streams_match_sequential(lib, gpu):
    import torch
    rng = np.random.default_rng(7)
    # 2:4 fp16
    A16 = _dev(wl.f16_normal(rng, (512, 1024)))
    v16, m16 = lib.w24_pack_f16(wl.prune24_magnitude(wl.f16_normal(rng, (1024, 512), 0.02)))
    v16, m16 = _dev(v16), _dev(m16.view(np.int32))
    # 2:4 int8, fp32 output
    A8 = _dev(wl.i8_uniform(rng, (600, 768)))
    v8, m8 = lib.w24_pack_i8(wl.prune24_magnitude(wl.i8_weights(rng, (768, 640))))
    v8, m8, sc = _dev(v8), _dev(m8.view(np.int32)), _dev(wl.f32_scales(rng, 640))
    # tile-wise fp16
    At = _dev(np.ascontiguousarray(wl.f16_normal(rng, (256, 768)).T))
    Wtw = wl.prune_tilewise(wl.f16_normal(rng, (768, 384), 0.02), 128, [0.3, 0.1, 0.6])
    ptw = lib.tw_pack_f16(Wtw, 128).to("cuda")
    # dense fp16
    Ad = _dev(wl.f16_normal(rng, (384, 512)))
    Wt = _dev(np.ascontiguousarray(wl.f16_normal(rng, (512, 256), 0.02).T))

    ops = [lambda out=None: lib.w24_gemm_f16(A16, v16, m16, out=out),
           lambda out=None: lib.w24_gemm_i8(A8, v8, m8, sc, out=out),
           lambda out=None: lib.tw_gemm_f16(At, ptw, out=out),
           lambda out=None: lib.dense_gemm_f16(Ad, Wt, out=out)]
    expect = [op() for op in ops]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in expect]
    streams = [torch.cuda.Stream() for _ in ops]
    for rep in range(5):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for _ in range(3):  # several launches per stream, interleaved across streams
            for s, op, o in zip(streams, ops, outs):
                with torch.cuda.stream(s):
                    op(out=o)
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, expect)):
            assert torch.equal(_bits(o), _bits(e)), f"op {i} differs on repetition {rep}"
