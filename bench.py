"""Benchmark of the structured-sparse weight GEMM on one MI355X.

Default run (the headline line): the 2:4 int8 GEMM at the ViT-Base MLP fc1
shape -- A [64*197 = 12608 x 768] int8, W [768 x 3072] int8 pruned 2:4 along
K, int32 accumulate, per-output-channel fp32 scale, fp32 output.  One step is
one w24_gemm_i8 launch over that batch with every input already resident in
HBM.  Input/output sets rotate over more than twice the 256 MB Infinity Cache
so every step streams from HBM.  The same-shape dense int8 GEMM (unpruned W)
is timed the same way for the speedup.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --all        # one JSON line per workload and kernel (table mode)

stdout carries exactly one JSON line in the default mode; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import shutil
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOPS/TOPS of sparse GEMM + speedup vs dense MFMA GEMM, same shape"
# Headline timing: after the W eager warm-up steps, the sparse and the dense
# graphs (K launches each) replay alternately for HEADLINE_WARM_S seconds so
# the power-managed shader clock settles at its sustained value, then
# HEADLINE_ROUNDS rounds each time one sparse replay and one dense replay
# (every replay a timed region of exactly K steps); medians are reported.
HEADLINE_ROUNDS = 25
HEADLINE_WARM_S = 1.5
# table mode: each graph replays this long (untimed) before its 5 timed replays
TABLE_WARM_S = 0.3
CACHE_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w24_gemm_i8_vit_base_fc1.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text):
    """C++ source without comments and with whitespace collapsed: edits to
    comments or layout do not change a kernel, so they keep its hash."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(main="gemm.hip"):
    """Hash of a kernel source and the shared header, code only (traffic
    counters are only reused while this matches)."""
    h = hashlib.sha256()
    for f in (main, "common.h"):
        src = open(os.path.join(ROOT, "structured_sparse_gemm_w24_amd", "csrc", "kernels", f)).read()
        h.update(_code_only(src).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-launch HBM bytes measured with rocprofv3 counters for the current kernel source, else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sha") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the stream the kernels are launched on.

    graph=True captures the `steps` launches into one HIP graph (the kernels
    allocate nothing and record no memsets, so they capture cleanly) and
    times its replay: the GPU then runs the launches back to back without
    host launch gaps, so the per-step time is the kernel's own duration plus
    the hardware's dispatch gap.  graph=False times eager launches from
    Python.  `reps` replays are timed one by one; the call returns the median
    per-step time and `stats` also gives p10 / p90 over the replays."""

    def __init__(self, torch, graph=True, reps=1, warm_s=0.0):
        self.torch = torch
        self.graph = graph
        self.reps = reps
        self.warm_s = warm_s  # untimed replays of the graph, in seconds, before the timed ones

    def __call__(self, fn, steps, warmup):
        return self.stats(fn, steps, warmup)["ms"]

    def stats(self, fn, steps, warmup, reps=None):
        torch = self.torch
        reps = reps or self.reps
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        if self.graph:
            stream = torch.cuda.Stream()
            stream.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for i in range(steps):
                        fn(i)
            torch.cuda.current_stream().wait_stream(stream)
            g.replay()  # warm replay
            torch.cuda.synchronize()
            # the shader clock is power-managed: keep the GPU busy until it settles
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < self.warm_s:
                g.replay()
                torch.cuda.synchronize()
            for _ in range(reps):
                s.record()
                g.replay()
                e.record()
                torch.cuda.synchronize()
                times.append(s.elapsed_time(e) / steps)
            del g
        else:
            for _ in range(reps):
                s.record()
                for i in range(steps):
                    fn(i)
                e.record()
                torch.cuda.synchronize()
                times.append(s.elapsed_time(e) / steps)
        t = np.array(times)
        return dict(ms=float(np.median(t)), p10=float(np.percentile(t, 10)), p90=float(np.percentile(t, 90)),
                    replays=reps)  # ms per call


def _gfx_clocks(node):
    """Current clocks (MHz) of the gfx domains (one per XCD) in amd-smi's JSON."""
    found = []
    if isinstance(node, dict):
        for k, v in node.items():
            if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict):
                try:
                    found.append(float(v["clk"]["value"]))
                except (TypeError, ValueError):
                    pass
            else:
                found += _gfx_clocks(v)
    elif isinstance(node, list):
        for v in node:
            found += _gfx_clocks(v)
    return found


def _gfx_activity(node):
    """gfx_activity (%) from amd-smi's usage metrics, or None."""
    if isinstance(node, dict):
        v = node.get("gfx_activity")
        if isinstance(v, dict) and "value" in v:
            try:
                return float(v["value"])
            except (TypeError, ValueError):
                return None
        for w in node.values():
            r = _gfx_activity(w)
            if r is not None:
                return r
    elif isinstance(node, list):
        for w in node:
            r = _gfx_activity(w)
            if r is not None:
                return r
    return None


def observed_sclk(torch, fn, steps, warm_s=2.0, max_s=15.0):
    """Shader clock read with `amd-smi metric -c` (run as a child process) while
    the GPU replays a graph of `steps` calls of fn back to back; the GPU is kept
    busy until amd-smi exits.  Returns the per-XCD clocks and their median, or
    None when amd-smi is missing or fails.  The clock is power-managed, so it
    is context for the roofline fraction, not a setting."""
    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                fn(i)
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    # the SMU's published metrics lag the load, so the GPU is kept busy for
    # warm_s before amd-smi samples, and until it exits
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
    proc = subprocess.Popen([exe, "metric", "-g", "0", "-c", "-u", "--json"], stdout=subprocess.PIPE,
                            stderr=subprocess.DEVNULL)
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < max_s:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
    del g
    try:
        out, _ = proc.communicate(timeout=5.0)
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return None
    if proc.returncode != 0:
        return None
    try:
        doc = json.loads(out)
    except ValueError:
        return None
    mhz = _gfx_clocks(doc)
    if not mhz:
        return None
    return {"median_mhz": float(np.median(mhz)), "per_xcd_mhz": mhz, "gfx_activity_pct": _gfx_activity(doc),
            "source": f"amd-smi metric -c -u, read after {warm_s:g} s of the timed graph replaying back to back"}


def paired_replays(torch, fns, steps, warmup, warm_s, rounds):
    """Times several step functions against each other under the same clock.

    Each fn gets `warmup` eager calls, then one HIP graph of `steps` calls;
    the graphs replay round-robin for warm_s seconds (untimed: the shader
    clock is power-managed and drops from its idle value during the first
    milliseconds of sustained load), then `rounds` timed rounds replay every
    graph once, in order, with HIP events on the replaying stream around each
    replay.  Returns per fn the median, p10 and p90 ms per step over the
    rounds.  Alternating the kernels gives each the same clock history, so
    their ratio does not depend on which was timed first."""
    for i in range(warmup):
        for fn in fns:
            fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graphs = []
    for fn in fns:
        stream.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    fn(i)
        torch.cuda.current_stream().wait_stream(stream)
        graphs.append(g)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    warm_replays = 0
    while time.perf_counter() - t0 < warm_s:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        warm_replays += 1
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in graphs]
    times = [[] for _ in graphs]
    for _ in range(rounds):
        for j, g in enumerate(graphs):
            s, e = ev[j]
            s.record()
            g.replay()
            e.record()
            torch.cuda.synchronize()
            times[j].append(s.elapsed_time(e) / steps)
    del graphs
    out = []
    for t in times:
        t = np.array(t)
        out.append(dict(ms=float(np.median(t)), p10=float(np.percentile(t, 10)), p90=float(np.percentile(t, 90)),
                        rounds=rounds, warm_replays=warm_replays))
    return out


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo, as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_time_ms(fn, reps=3):
    """Median wall time of a host call (the pack stage runs offline, outside the
    timed GPU region; it is reported beside it)."""
    ts = []
    out = None
    for _ in range(reps):
        t0 = time.perf_counter()
        out = fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts)) * 1e3, out


def rotation(bytes_per_set):
    return max(2, int(np.ceil(2 * CACHE_BYTES / max(1, bytes_per_set))))


# ---------------------------------------------------------------- vendor 2:4 baseline
_VENDOR = []


# ---------------------------------------------------------------- measured matrix-core rates
_PEAK = []
# (name, kind of the probe, dense-equivalent operations per instruction)
PEAK_KINDS = (("dense_f16", 0, 32768), ("w24_f16", 1, 65536), ("dense_i8", 2, 65536), ("w24_i8", 3, 131072))


def mfma_peak_measured(torch, iters=1000, blocks=1536, reps=5, warm_s=0.3):
    """The rate this device sustains for each matrix instruction the GEMMs use
    (dense-equivalent TFLOP/s or TOPS), from libssg_peak.so (bench only: every
    wave issues the instruction back to back on four independent accumulators;
    1536 workgroups of 256 threads, `iters` x 4 instructions per wave).  Each kind
    runs warm for `warm_s` seconds, then `reps` launches are timed with HIP events
    on the current stream and the median is kept.  None when the probe library
    is missing or fails."""
    if _PEAK:
        return _PEAK[0]
    import ctypes as ct
    path = os.path.join(ROOT, "structured_sparse_gemm_w24_amd", "libssg_peak.so")
    res = None
    if os.path.exists(path):
        try:
            lib = ct.CDLL(path)
            fn = lib.ssg_bench_mfma_peak
            fn.restype = ct.c_int
            fn.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            st = torch.cuda.current_stream()
            res = {}
            for name, kind, ops in PEAK_KINDS:
                def launch():
                    rc = fn(kind, iters, blocks, ct.c_void_p(out.data_ptr()), ct.c_void_p(st.cuda_stream))
                    if rc:
                        raise RuntimeError(f"probe launch status {rc}")
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < warm_s:
                    launch()
                    torch.cuda.synchronize()
                times = []
                for _ in range(reps):
                    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s0.record()
                    launch()
                    s1.record()
                    torch.cuda.synchronize()
                    times.append(s0.elapsed_time(s1) * 1e-3)
                res[name] = blocks * 4 * iters * 4 * ops / float(np.median(times)) / 1e12
            res["unit"] = "dense-equivalent TFLOP/s (fp16) / TOPS (int8)"
            res["source"] = (f"libssg_peak.so: {blocks} workgroups x 4 waves, each issuing {iters * 4} back-to-back "
                             f"instructions on 4 accumulators; median of {reps} launches after {warm_s:g} s warm")
        except (OSError, RuntimeError, AttributeError) as e:
            log(f"matrix-core rate probe not used: {e}")
            res = None
    _PEAK.append(res)
    return res


def measured_mfma_frac(d, peak):
    """For a table line of a 2:4 or tile-wise GEMM: the fraction of the measured
    matrix-core rate its kernel reached (ideal time at the measured rate / time)."""
    if not peak or "t_sparse_ms" not in d:
        return None
    w = d.get("workload", "")
    if "tflops_dense_eq" in d and w.endswith("_w24_f16"):
        return d["tflops_dense_eq"] / peak["w24_f16"]
    if "tops_dense_eq" in d and "_w24_i8" in w:
        return d["tops_dense_eq"] / peak["w24_i8"]
    if "tflops_nonzero" in d and w.endswith("_tw_f16"):  # the tile-wise kernel runs dense instructions
        return d["tflops_nonzero"] / peak["dense_f16"]
    return None


def vendor_lib():
    """AMD's hipSPARSELt through libssg_vendor.so (built beside libssg when the
    hipSPARSELt headers are installed), or None.  Bench only: the product never
    loads it."""
    if not _VENDOR:
        import ctypes as ct
        path = os.path.join(ROOT, "structured_sparse_gemm_w24_amd", "libssg_vendor.so")
        v = None
        if os.path.exists(path):
            try:
                v = ct.CDLL(path)
            except OSError as e:
                log(f"vendor baseline not loaded: {e}")
                _VENDOR.append(None)
                return None
            v.vsl_create.restype = ct.c_void_p
            v.vsl_create.argtypes = [ct.c_int] * 5 + [ct.c_float] + [ct.c_void_p] * 4
            v.vsl_run.restype = ct.c_int
            v.vsl_run.argtypes = [ct.c_void_p] * 4
            v.vsl_destroy.argtypes = [ct.c_void_p]
            v.vsl_last_error.restype = ct.c_char_p
        _VENDOR.append(v)
    return _VENDOR[0]


def vendor_w24_time(torch, kind, Wp, sets, M, N, K, C_ours, steps, warmup, timer):
    """Times hipSPARSELt's 2:4 GEMM on the same operands: kind 0 fp16 in / fp16
    out, kind 1 int8 in / fp16 out.  The vendor output is alpha * product with
    a scalar alpha: 1 for fp16, 2^-12 for int8 (the raw accumulators exceed
    the fp16 range), where the int8 kernel beside it applies a per-channel
    scale vector.  C_ours is the unscaled product.  Both operand orientations are
    planned (algorithm search on each) and the faster is reported.  The weight
    is compressed once; A and C rotate over `sets` like the other kernels'.
    Every plan's first result is checked against alpha * C_ours (C_ours: this
    library's unscaled product for sets[0]) before it is timed.  Returns {} when the library is absent."""
    v = vendor_lib()
    if v is None:
        return {}
    dev = torch.device("cuda")
    R = len(sets)
    W_t = torch.from_numpy(np.ascontiguousarray(Wp)).to(dev)
    best, notes = None, []
    alpha = 1.0 if kind == 0 else 2.0 ** -12
    ref = C_ours.float() * alpha
    for rowmajor in (0, 1):
        W_o = W_t if rowmajor == 0 else W_t.t().contiguous()
        stream = torch.cuda.current_stream().cuda_stream
        plan = v.vsl_create(kind, M, N, K, rowmajor, alpha, W_o.data_ptr(), sets[0]["A"].data_ptr(),
                            sets[0]["C"].data_ptr(), stream)
        if not plan:
            notes.append(f"orientation {rowmajor}: {v.vsl_last_error().decode()}")
            continue
        try:
            Cv = torch.empty(M * N, dtype=torch.float16, device=dev)
            if v.vsl_run(plan, sets[0]["A"].data_ptr(), Cv.data_ptr(), stream) != 0:
                notes.append(f"orientation {rowmajor}: {v.vsl_last_error().decode()}")
                continue
            torch.cuda.synchronize()
            got = (Cv.view(M, N) if rowmajor == 0 else Cv.view(N, M).t()).float()
            err = float((got - ref).abs().max() / ref.abs().max().clamp_min(1e-30))
            if not err < 1e-2:
                notes.append(f"orientation {rowmajor}: result differs (max rel err {err:.3g})")
                continue

            def fn(i, plan=plan):
                d = sets[i % R]
                rc = v.vsl_run(plan, d["A"].data_ptr(), d["C"].data_ptr(), torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError(v.vsl_last_error().decode())

            mode = "graph"
            try:
                t = timer(fn, steps, warmup)
            except RuntimeError as e:
                torch.cuda.synchronize()
                mode = "eager"
                notes.append(f"orientation {rowmajor}: graph capture failed ({e}); timed eagerly")
                t = Timer(torch, graph=False, reps=timer.reps)(fn, steps, warmup)
            if best is None or t < best[0]:
                best = (t, rowmajor, mode, err)
        finally:
            torch.cuda.synchronize()
            v.vsl_destroy(plan)
    out = {"vendor_notes": notes} if notes else {}
    if best is not None:
        out.update(t_vendor_sparse_ms=best[0], vendor_orientation=["col-major", "row-major"][best[1]],
                   vendor_timing=best[2], vendor_max_rel_err=best[3])
    return out


# ---------------------------------------------------------------- workloads
def w24_i8_case(torch, ssg, perf, c, steps, warmup, timer, rotate=True, with_f16_dense=False, paired=None):
    """2:4 and dense int8 GEMMs at c's shape.  paired = (warm_s, rounds): time
    both with paired_replays (the headline) instead of the table timer."""
    dev = torch.device("cuda")
    M, K, N = c["M"], c["K"], c["N"]
    t_pack, (vals, meta) = host_time_ms(lambda: ssg.w24_pack_i8(c["Wp"]))
    sets_bytes = perf.w24_bytes(M, N, K, 1, 1, 4, scale=True)
    R = rotation(sets_bytes) if rotate else 1
    A0 = torch.from_numpy(c["A"]).to(dev)
    sets = []
    for r in range(R):
        sets.append(dict(A=A0.clone() if r else A0, vals=torch.from_numpy(vals).to(dev),
                         meta=torch.from_numpy(meta.view(np.int32)).to(dev),
                         scale=torch.from_numpy(c["scale"]).to(dev),
                         C=torch.empty((M, N), dtype=torch.float32, device=dev),
                         Wt=torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)))
    sp = lambda i: ssg.w24_gemm_i8(sets[i % R]["A"], sets[i % R]["vals"], sets[i % R]["meta"],
                                   sets[i % R]["scale"], out=sets[i % R]["C"])
    de = lambda i: ssg.dense_gemm_i8(sets[i % R]["A"], sets[i % R]["Wt"], sets[i % R]["scale"],
                                     out=sets[i % R]["C"])
    if paired is not None:
        st, sd = paired_replays(torch, [sp, de], steps, warmup, *paired)
        t_de = sd["ms"]
        extra = dict(t_dense_p10_ms=sd["p10"], t_dense_p90_ms=sd["p90"], rounds=st["rounds"],
                     warm_replays=st["warm_replays"])
    else:
        st = timer.stats(sp, steps, warmup)
        t_de = timer(de, steps, warmup)
        extra = {}
    out = dict(t_sparse_ms=st["ms"], t_sparse_p10_ms=st["p10"], t_sparse_p90_ms=st["p90"], t_dense_ms=t_de,
               rotate_sets=R, t_pack_host_ms=t_pack, sets=sets, sp=sp, **extra,
               k_splits=ssg.splitk_suggest(ssg.SSG_KIND_W24_I8, M, N, K),
               k_splits_dense=ssg.splitk_suggest(ssg.SSG_KIND_DENSE_I8, M, N, K))
    if with_f16_dense:
        # the same shape through the fp16 dense kernel (int8 values are exact in fp16)
        for d in sets:
            d["A16"] = d["A"].to(torch.float16)
            d["Wt16"] = d["Wt"].to(torch.float16)
            d["C16"] = torch.empty((M, N), dtype=torch.float16, device=dev)
        d16 = lambda i: ssg.dense_gemm_f16(sets[i % R]["A16"], sets[i % R]["Wt16"], out=sets[i % R]["C16"])
        out["t_dense_f16_ms"] = timer(d16, steps, warmup)
        for d in sets:
            del d["A16"], d["Wt16"], d["C16"]
    return out


def w24_i8_out_case(torch, ssg, perf, c, out_type, steps, warmup, timer, rotate=True, vendor=False):
    """2:4 and dense int8 GEMMs with the lower-traffic epilogue (fp16 or int8 output)."""
    dev = torch.device("cuda")
    M, K, N = c["M"], c["K"], c["N"]
    ob = {"f16": 2, "i8": 1}[out_type]
    odt = {"f16": torch.float16, "i8": torch.int8}[out_type]
    vals, meta = ssg.w24_pack_i8(c["Wp"])
    R = rotation(perf.w24_bytes(M, N, K, 1, 1, ob, scale=True)) if rotate else 1
    A0 = torch.from_numpy(c["A"]).to(dev)
    sets = [dict(A=A0.clone() if r else A0, vals=torch.from_numpy(vals).to(dev),
                 meta=torch.from_numpy(meta.view(np.int32)).to(dev), scale=torch.from_numpy(c["scale"]).to(dev),
                 C=torch.empty((M, N), dtype=odt, device=dev),
                 Wt=torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)) for r in range(R)]
    sp = lambda i: ssg.w24_gemm_i8_out(sets[i % R]["A"], sets[i % R]["vals"], sets[i % R]["meta"],
                                       sets[i % R]["scale"], out_type=out_type, out=sets[i % R]["C"])
    de = lambda i: ssg.dense_gemm_i8_out(sets[i % R]["A"], sets[i % R]["Wt"], sets[i % R]["scale"],
                                         out_type=out_type, out=sets[i % R]["C"])
    st = timer.stats(sp, steps, warmup)
    out = dict(t_sparse_ms=st["ms"], t_sparse_p10_ms=st["p10"], t_sparse_p90_ms=st["p90"],
               t_dense_ms=timer(de, steps, warmup), rotate_sets=R, out_bytes=ob)
    if vendor and out_type == "f16":
        # the vendor call applies no channel scale: its check is against the raw accumulators
        acc = ssg.w24_gemm_i8_out(sets[0]["A"], sets[0]["vals"], sets[0]["meta"], None, out_type="i32")
        out.update(vendor_w24_time(torch, 1, c["Wp"], sets, M, N, K, acc, steps, warmup, timer))
    return out


def tw_i8_case(torch, ssg, perf, c, out_type, steps, warmup, timer, rotate=True):
    """int8 tile-wise GEMM (fp16 or int8 output) and the dense int8 GEMM with the same epilogue."""
    dev = torch.device("cuda")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    odt = {"f16": torch.float16, "i8": torch.int8}[out_type]
    ob = {"f16": 2, "i8": 1}[out_type]
    host = ssg.tw_pack_i8(c["Wp"], G)
    R = rotation(M * K + M * N * ob + host.vals.size) if rotate else 1
    A = torch.from_numpy(c["A"]).to(dev)
    sets = [dict(A=A, At=A.t().contiguous(), packed=host.to(dev), scale=torch.from_numpy(c["scale"]).to(dev),
                 C=torch.empty((M, N), dtype=odt, device=dev),
                 Wt=torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)) for _ in range(R)]
    sp = lambda i: ssg.tw_gemm_i8(sets[i % R]["At"], sets[i % R]["packed"], sets[i % R]["scale"], out_type=out_type,
                                  out=sets[i % R]["C"])
    de = lambda i: ssg.dense_gemm_i8_out(sets[i % R]["A"], sets[i % R]["Wt"], sets[i % R]["scale"],
                                         out_type=out_type, out=sets[i % R]["C"])
    nnz = int((np.diff(host.k_ptr) * np.diff(host.n_ptr)).sum())
    st = timer.stats(sp, steps, warmup)
    return dict(t_sparse_ms=st["ms"], t_sparse_p10_ms=st["p10"], t_sparse_p90_ms=st["p90"],
                t_dense_ms=timer(de, steps, warmup), rotate_sets=R, ops=perf.tw_ops(M, nnz))


def w24_f16_case(torch, ssg, perf, c, steps, warmup, timer, rotate=True, vendor=False):
    dev = torch.device("cuda")
    M, K, N = c["M"], c["K"], c["N"]
    t_pack, (vals, meta) = host_time_ms(lambda: ssg.w24_pack_f16(c["Wp"]))
    R = rotation(perf.w24_bytes(M, N, K, 2, 2, 2)) if rotate else 1
    sets = [dict(A=torch.from_numpy(c["A"]).to(dev), vals=torch.from_numpy(vals).to(dev),
                 meta=torch.from_numpy(meta.view(np.int32)).to(dev),
                 C=torch.empty((M, N), dtype=torch.float16, device=dev),
                 Wt=torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)) for _ in range(R)]
    sp = lambda i: ssg.w24_gemm_f16(sets[i % R]["A"], sets[i % R]["vals"], sets[i % R]["meta"], out=sets[i % R]["C"])
    de = lambda i: ssg.dense_gemm_f16(sets[i % R]["A"], sets[i % R]["Wt"], out=sets[i % R]["C"])
    tm = lambda i: torch.matmul(sets[i % R]["A"], sets[i % R]["Wt"].T)
    st = timer.stats(sp, steps, warmup)
    out = dict(t_sparse_ms=st["ms"], t_sparse_p10_ms=st["p10"], t_sparse_p90_ms=st["p90"],
               t_dense_ms=timer(de, steps, warmup), t_torch_ms=timer(tm, steps, warmup), rotate_sets=R,
               t_pack_host_ms=t_pack, k_splits=ssg.splitk_suggest(ssg.SSG_KIND_W24_F16, M, N, K),
               k_splits_dense=ssg.splitk_suggest(ssg.SSG_KIND_DENSE_F16, M, N, K))
    if vendor:
        sp(0)
        out.update(vendor_w24_time(torch, 0, c["Wp"], sets, M, N, K, sets[0]["C"].clone(), steps, warmup, timer))
    return out


def tw_case(torch, ssg, perf, c, steps, warmup, timer, rotate=True, extras=True):
    dev = torch.device("cuda")
    M, K, N, G = c["M"], c["K"], c["N"], c["G"]
    t_pack, host = host_time_ms(lambda: ssg.tw_pack_f16(c["Wp"], G))
    union = int(np.unique(host.offset_k).size)
    bytes_ = perf.tw_bytes(M, N, union, host.vals.size, host.offset_k.size, host.offset_n.size, host.T)
    R = rotation(bytes_ + M * K * 2) if rotate else 1
    A = torch.from_numpy(c["A"]).to(dev)
    sets = [dict(A=A, At=ssg.ssg_transpose_f16(A), packed=host.to(dev),
                 C=torch.empty((M, N), dtype=torch.float16, device=dev),
                 Wt=torch.from_numpy(np.ascontiguousarray(c["W"].T)).to(dev)) for _ in range(R)]
    sp = lambda i: ssg.tw_gemm_f16(sets[i % R]["At"], sets[i % R]["packed"], out=sets[i % R]["C"])
    tr = lambda i: ssg.ssg_transpose_f16(sets[i % R]["A"], out=sets[i % R]["At"])
    de = lambda i: ssg.dense_gemm_f16(sets[i % R]["A"], sets[i % R]["Wt"], out=sets[i % R]["C"])
    tm = lambda i: torch.matmul(sets[i % R]["A"], sets[i % R]["Wt"].T)
    nnz = int((np.diff(host.k_ptr) * np.diff(host.n_ptr)).sum())
    st = timer.stats(sp, steps, warmup)
    out = dict(t_sparse_ms=st["ms"], t_sparse_p10_ms=st["p10"], t_sparse_p90_ms=st["p90"],
               t_transpose_ms=timer(tr, steps, warmup), t_dense_ms=timer(de, steps, warmup),
               t_torch_ms=timer(tm, steps, warmup), rotate_sets=R, bytes=bytes_, ops=perf.tw_ops(M, nnz),
               union_rows=union, t_pack_host_ms=t_pack, max_kept_columns=host.max_nt,
               tw_kernel="narrow (SSG_TW_NARROW)" if host.narrow() and G <= 128 else "general")
    if not extras:
        return out
    # fused transpose: the same GEMM writing Ct [N][M], the next tile-wise layer's At
    for d in sets:
        d["Ct"] = torch.empty((N, M), dtype=torch.float16, device=dev)
    fu = lambda i: ssg.tw_gemm_f16_ex(sets[i % R]["At"], sets[i % R]["packed"], out_t=True, out=sets[i % R]["Ct"])
    t_fused = timer(fu, steps, warmup)
    # the slides' "without transpose" case: row-major A gathered as scattered elements
    nt_ = lambda i: ssg.tw_gemm_f16_ex(sets[i % R]["A"], sets[i % R]["packed"], a_rowmajor=True, out=sets[i % R]["C"])
    t_no_transpose = timer(nt_, steps, warmup)
    # the slides' multi-stream schedule: one launch per tile over 4 streams
    streams = [torch.cuda.Stream() for _ in range(4)]
    ms = lambda i: ssg.tw_gemm_f16_streams(sets[i % R]["At"], sets[i % R]["packed"], streams, out=sets[i % R]["C"])
    try:
        t_ms, ms_timing = timer(ms, steps, warmup), "graph"
    except RuntimeError:
        t_ms, ms_timing = Timer(torch, graph=False)(ms, steps, warmup), "eager"
    out.update(t_fused_transposed_out_ms=t_fused, t_no_transpose_ms=t_no_transpose, t_multistream4_ms=t_ms,
               multistream_timing=ms_timing)
    return out


# ---------------------------------------------------------------- cpu baseline
def cpu_baseline(c, perf, budget_s=12.0, one_core_rows=1024, gpu_out=None):
    """The oracle as it stands, on the host cores, over a bounded number of full
    repetitions; then on one core over the first `one_core_rows` token rows
    (median of 3), the same GEMM restricted to a slice of A.  gpu_out (host
    copy of a timed launch's output) is compared with the first repetition's
    result bit for bit."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    reps, t0, ref = 0, time.perf_counter(), None
    while True:
        C_ref = oracle.ref_gemm_i8(c["A"], c["Wp"], c["scale"])
        if ref is None:
            ref = C_ref
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    nz, _ = perf.w24_ops(c["M"], c["N"], c["K"])
    out = {"value": nz * reps / el / 1e12, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
           "sample": f"full {c['M']}x{c['K']}x{c['N']} int8 GEMM + epilogue (numpy float64 BLAS), "
                     f"{reps} repetition(s), {el:.1f} s; host CPU {host_cpu_model()}, {os.cpu_count()} "
                     f"logical CPUs visible"}
    if gpu_out is not None:
        diff = np.abs(gpu_out.astype(np.float64) - ref.astype(np.float64))
        out["parity"] = {"what": "output of a timed launch vs the oracle's first repetition, every element",
                         "elements": int(ref.size), "bit_exact": bool(np.array_equal(gpu_out.view(np.uint32),
                                                                                      ref.view(np.uint32))),
                         "max_abs_diff": float(np.nanmax(diff)) if diff.size else 0.0}
    if threadpool_limits is not None:
        rows = min(one_core_rows, c["M"])
        A = np.ascontiguousarray(c["A"][:rows])
        ts = []
        with threadpool_limits(limits=1):
            for _ in range(3):
                t1 = time.perf_counter()
                oracle.ref_gemm_i8(A, c["Wp"], c["scale"])
                ts.append(time.perf_counter() - t1)
        nz1, _ = perf.w24_ops(rows, c["N"], c["K"])
        out["one_core"] = {"value": nz1 / float(np.median(ts)) / 1e12, "unit": "TOPS", "cores": 1,
                           "sample": f"first {rows} token rows of the same GEMM, median of 3"}
    return out


# ---------------------------------------------------------------- main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="table mode: every workload and kernel")
    ap.add_argument("--workloads", default="",
                    help="table mode: comma list from " + ",".join(WORKLOADS + SUB_WORKLOADS) +
                         " (vit_large:<gemm>: one layer-0 GEMM; default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the shader-clock reading (2 s of extra replays; for profiled runs)")
    ap.add_argument("--no-tw-extras", action="store_true",
                    help="table mode: time only the grouped tile-wise kernel (not the fused, row-major-A "
                         "and multi-stream variants)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="table mode: skip the vendor 2:4 library (hipSPARSELt) beside the 2:4 kernels")
    ap.add_argument("--warm", action="store_true", help="one input set (cache-resident) instead of rotating")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a replayed HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain device copy of known size (for scaling HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="summarise rocprofv3 CSV output under DIR into --out (no GPU needed)")
    ap.add_argument("--kernel", default="gemm_kernel<3", help="kernel-name substring for --summarize-profile")
    ap.add_argument("--kernel-source", default="gemm.hip",
                    help="kernel source file whose hash the --summarize-profile summary records")
    ap.add_argument("--out", help="summary file for --summarize-profile")
    ap.add_argument("--command", default="", help="the profiled command line, recorded in the summary")
    ap.add_argument("--profile-steps", type=int, default=20, help="--steps of the profiled command (dispatch groups)")
    ap.add_argument("--profile-warmup", type=int, default=5, help="--warmup of the profiled command")
    ap.add_argument("--bench-log", help="stdout of the profiled command (its bench line is quoted in the summary)")
    ap.add_argument("--k-stages", type=int, default=0,
                    help="--summarize-profile: K stages per output tile, to report cycles per K-stage")
    a = ap.parse_args(argv)
    if a.summarize_profile:
        return summarize_profile(a)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}): the sparse GEMM is timed on one "
              "GPU's share of the work, and sharding it across GPUs is not implemented", file=sys.stderr)
        return 2

    import torch

    import structured_sparse_gemm_w24_amd as ssg
    import workloads as wl
    from structured_sparse_gemm_w24_amd import perf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    timer = Timer(torch, graph=not a.eager)
    if a.copy_calibration:
        return copy_calibration(torch, a.steps)
    log("device", ssg.ssg_device_arch())
    if a.all:
        return table(a, torch, ssg, perf, wl, timer)

    c = wl.make_vit_base_fc1_i8()
    M, K, N = c["M"], c["K"], c["N"]
    log(f"workload vit_base_mlp_fc1 2:4 int8 {M}x{K}x{N}, steps {a.steps}, warmup {a.warmup}")
    r = w24_i8_case(torch, ssg, perf, c, a.steps, a.warmup, timer, rotate=not a.warm,
                    paired=(HEADLINE_WARM_S, HEADLINE_ROUNDS))
    log(f"sparse {r['t_sparse_ms'] * 1e3:.1f} us/step (p10 {r['t_sparse_p10_ms'] * 1e3:.1f}, "
        f"p90 {r['t_sparse_p90_ms'] * 1e3:.1f}), dense {r['t_dense_ms'] * 1e3:.1f} us/step")
    step = r["sp"]
    t_eager = Timer(torch, graph=False, reps=5)(step, a.steps, a.warmup)
    sclk = observed_sclk(torch, step, a.steps) if not (a.eager or a.no_sclk) else None
    nz, de = perf.w24_ops(M, N, K)
    t = r["t_sparse_ms"] / 1e3
    bytes_ = perf.w24_bytes(M, N, K, 1, 1, 4, scale=True)
    achieved = bytes_ / t / 1e9
    traffic = read_traffic()
    peak = mfma_peak_measured(torch) if not a.eager else None
    line = {
        "metric": METRIC,
        "value": nz / t / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": r["t_sparse_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded; ViT-Base MLP fc1 shape, int8 U[-127,127] activations, "
                "round(N(0,32)) weights 2:4-pruned by magnitude, U(1e-3,1e-2) scales)",
        "config": {"workload": "vit_base_mlp_fc1_w24_i8", "M": M, "K": K, "N": N,
                   "pattern": "2:4 along K", "accumulate": "int32", "output": "fp32 (per-channel scale)",
                   "inputs": "rotating HBM-resident sets" if not a.warm else "one cache-resident set",
                   "rotate_sets": r["rotate_sets"]},
        "dense_equivalent_tops": de / t / 1e12,
        "speedup_vs_dense": perf.speedup(r["t_dense_ms"], r["t_sparse_ms"]),
        "dense_i8_ms": r["t_dense_ms"],
        "pack_host_ms": r["t_pack_host_ms"],
        "timing": f"{a.warmup} eager warm-up steps per kernel; HIP graphs of the {a.steps} steps of the sparse "
                  f"and of the dense kernel replayed alternately for {HEADLINE_WARM_S:g} s (untimed, "
                  f"{r['warm_replays']} pairs) so the power-managed clock settles; then {r['rounds']} rounds "
                  f"of one sparse and one dense replay, HIP events on the replay stream around each "
                  f"replay; ms_per_step = median sparse replay / {a.steps} (p10 / p90 beside)",
        "rounds": r["rounds"],
        "ms_per_step_p10": r["t_sparse_p10_ms"],
        "ms_per_step_p90": r["t_sparse_p90_ms"],
        "dense_i8_ms_p10": r["t_dense_p10_ms"],
        "dense_i8_ms_p90": r["t_dense_p90_ms"],
        "eager_ms_per_step": t_eager,
        "sclk": sclk,
        "roofline": perf.roofline(achieved, perf.PEAK_HBM_GBS, "GB/s", "hbm", traffic),
        "mfma_peak_measured": peak,
        "mfma_frac_of_measured_peak": (de / t / 1e12 / peak["w24_i8"]) if peak else None,
        "cpu_baseline": None,
    }
    # one more launch of the timed step on set 0 (the dense timing shares the
    # output buffers), copied out for the oracle's check
    C_gpu = None
    if not a.no_cpu:
        step(0)
        torch.cuda.synchronize()
        C_gpu = r["sets"][0]["C"].cpu().numpy()
    del r
    torch.cuda.empty_cache()
    if not a.no_cpu:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(c, perf, gpu_out=C_gpu)
    print(json.dumps(line), flush=True)
    return 0


COPY_BYTES = 256 << 20


def copy_calibration(torch, steps):
    """A plain device-to-device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES) per launch."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(1, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {steps} copies of {COPY_BYTES} bytes")
    return 0


def _csv_rows(root, suffix):
    import csv
    rows = []
    for d, _, files in os.walk(root):
        for f in files:
            if f.endswith(suffix):
                with open(os.path.join(d, f)) as fh:
                    rows += list(csv.DictReader(fh))
    return rows


def summarize_profile(a):
    """Writes a short text summary of rocprofv3 CSV output found under DIR:
    DIR/trace (--kernel-trace --stats), DIR/fetch and DIR/write (--pmc FETCH_SIZE,
    --pmc WRITE_SIZE on the same command), DIR/copy_fetch and DIR/copy_write (the
    same counters on --copy-calibration), optionally DIR/mfma (--pmc
    SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE).  The counters are KiB per dispatch; the
    copy of COPY_BYTES gives the scale from counted to true bytes."""
    root = a.summarize_profile
    out = []
    for r in _csv_rows(os.path.join(root, "trace"), "kernel_stats.csv"):
        out.append(f"kernel: {r.get('Name', '')[:160]}")
        out.append(f"  calls {r.get('Calls')}  avg_ns {r.get('AverageNs')}  min_ns {r.get('MinNs')}  "
                   f"max_ns {r.get('MaxNs')}  share_pct {r.get('Percentage')}")

    def counter(sub, cname, match):
        vals = []
        for r in _csv_rows(os.path.join(root, sub), "counter_collection.csv"):
            name = r.get("Kernel_Name", "")
            if r.get("Counter_Name") == cname and match(name):
                try:
                    vals.append(float(r.get("Counter_Value")))
                except (TypeError, ValueError):
                    pass
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    is_target = lambda n: a.kernel in n
    is_copy = lambda n: "copy" in n.lower() and "elementwise" not in n.lower()
    # the target's dispatches in launch order: the profiled bench does `warmup`
    # eager calls, then groups of `steps` (one graph replay or one eager
    # repetition each), so per-group medians show the timed replays apart
    # from the warm-up, and the clock's drift under sustained load
    tr = [r for r in _csv_rows(os.path.join(root, "trace"), "kernel_trace.csv") if is_target(r.get("Kernel_Name", ""))]
    if tr:
        tr.sort(key=lambda r: int(r["Start_Timestamp"]))
        d = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr]) / 1e3
        out.append(f"target '{a.kernel}': {d.size} dispatches, mean {d.mean():.1f} us, median {np.median(d):.1f} us")
        w, st = max(0, a.profile_warmup), max(1, a.profile_steps)
        groups = [d[:w]] + [d[i:i + st] for i in range(w, d.size, st)]
        shown = [g for g in groups if g.size][:40]
        out.append(f"  per-group median us (warm-up {w}, then groups of {st}; first {len(shown)} of "
                   f"{sum(1 for g in groups if g.size)}): " + " ".join(f"{np.median(g):.1f}" for g in shown))
    if a.bench_log and os.path.exists(a.bench_log):
        lines = [ln for ln in open(a.bench_log) if ln.startswith("{")]
        for ln in lines:
            j = json.loads(ln)
            if "ms_per_step" in j:
                out.append(f"bench line of the profiled command: ms_per_step {j['ms_per_step'] * 1e3:.1f} us "
                           f"(p10 {j.get('ms_per_step_p10', float('nan')) * 1e3:.1f}, "
                           f"p90 {j.get('ms_per_step_p90', float('nan')) * 1e3:.1f}), "
                           f"dense {j.get('dense_i8_ms', float('nan')) * 1e3:.1f} us")
            elif "t_sparse_ms" in j:
                out.append(f"bench line of the profiled command: {j.get('workload')} t_sparse {j['t_sparse_ms'] * 1e3:.1f} us, "
                           f"t_dense {j.get('t_dense_ms', float('nan')) * 1e3:.1f} us")
    tf, ntf = counter("fetch", "FETCH_SIZE", is_target)
    tw, ntw = counter("write", "WRITE_SIZE", is_target)
    cf, ncf = counter("copy_fetch", "FETCH_SIZE", is_copy)
    cw, ncw = counter("copy_write", "WRITE_SIZE", is_copy)
    out.append(f"target '{a.kernel}': FETCH_SIZE {tf} KiB ({ntf} dispatches), WRITE_SIZE {tw} KiB ({ntw})")
    busy, nb = counter("mfma", "SQ_VALU_MFMA_BUSY_CYCLES", is_target)
    gui, ng = counter("mfma", "GRBM_GUI_ACTIVE", is_target)
    if busy is not None and gui:
        # MFMA busy cycles are summed over every SIMD (a 32x32 sparse or
        # 32x32x16 dense instruction counts 32 cycles, its issue interval at
        # peak); GRBM_GUI_ACTIVE is summed over the 8 XCDs, each with 32 CUs x
        # 4 SIMDs, so the fraction of the matrix-core peak at the running clock
        # is busy / (GUI_ACTIVE x 128)
        out.append(f"target '{a.kernel}': SQ_VALU_MFMA_BUSY_CYCLES {busy:.0f}, GRBM_GUI_ACTIVE {gui:.0f} "
                   f"({nb} dispatches); MFMA busy fraction = busy / (GUI_ACTIVE x 128) = {busy / (gui * 128):.3f}")
        if a.k_stages:
            # one round of output tiles (at most one workgroup per CU): the
            # kernel's cycles per XCD over its K stages
            out.append(f"  cycles per K-stage (GRBM_GUI_ACTIVE / 8 XCDs / {a.k_stages} stages, one round of "
                       f"tiles): {gui / 8 / a.k_stages:.0f}")
    out.append(f"copy of {COPY_BYTES} B: FETCH_SIZE {cf} KiB ({ncf}), WRITE_SIZE {cw} KiB ({ncw})")
    if None not in (cf, cw, tf, tw) and cf > 0 and cw > 0:
        kf, kw = COPY_BYTES / (cf * 1024), COPY_BYTES / (cw * 1024)
        out.append(f"scale (true bytes per counted byte): fetch {kf:.4f} write {kw:.4f}")
        out.append(f"kernel_sha: {kernel_hash(a.kernel_source)}")
        out.append(f"hbm_read_bytes_per_launch: {tf * 1024 * kf:.0f}")
        out.append(f"hbm_write_bytes_per_launch: {tw * 1024 * kw:.0f}")
        out.append(f"hbm_bytes_per_launch: {tf * 1024 * kf + tw * 1024 * kw:.0f}")
    text = "\n".join([f"# rocprofv3 summary; command: {a.command}"] + out) + "\n"
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text)
    return 0


def vit_large_stack(torch, ssg, perf, wl, dtype, timer, steps_gemm=20, passes=3, layers=24):
    """The ViT-Large stack: `layers` x (qkv, proj, fc1, fc2), each GEMM with its own
    2:4 weight and its own A, all resident in HBM.  Two views of "sum of GEMM time":
    the sum over the GEMMs of each one's own graph-timed time (a GEMM repeated on
    its own data, so its inputs are cache-warm), and one back-to-back replay of all
    launches in layer order (the stack's working set is far larger than the
    Infinity Cache, so this one streams weights and activations from HBM)."""
    dev = torch.device("cuda")
    odt = torch.float16 if dtype == "f16" else torch.float32
    gemms, outs = [], {}
    t0 = time.perf_counter()
    for g in wl.vit_large_layers(dtype, layers=layers):
        vals, meta = (ssg.w24_pack_f16 if dtype == "f16" else ssg.w24_pack_i8)(g["Wp"])
        d = dict(shape=g["name"].rsplit("_", 1)[1], M=g["M"], K=g["K"], N=g["N"],
                 A=torch.from_numpy(g["A"]).to(dev), vals=torch.from_numpy(vals).to(dev),
                 meta=torch.from_numpy(meta.view(np.int32)).to(dev),
                 Wt=torch.from_numpy(np.ascontiguousarray(g["W"].T)).to(dev),
                 scale=torch.from_numpy(g["scale"]).to(dev) if dtype == "i8" else None)
        key = (g["M"], g["N"])
        if key not in outs:
            outs[key] = torch.empty(key, dtype=odt, device=dev)
        d["C"] = outs[key]
        gemms.append(d)
        if len(gemms) % 16 == 0:
            log(f"ViT-Large {dtype} stack: {len(gemms)} GEMMs generated and uploaded ({time.perf_counter() - t0:.0f} s)")

    def sparse(d):
        if dtype == "f16":
            return ssg.w24_gemm_f16(d["A"], d["vals"], d["meta"], out=d["C"])
        return ssg.w24_gemm_i8(d["A"], d["vals"], d["meta"], d["scale"], out=d["C"])

    def dense(d):
        if dtype == "f16":
            return ssg.dense_gemm_f16(d["A"], d["Wt"], out=d["C"])
        return ssg.dense_gemm_i8(d["A"], d["Wt"], d["scale"], out=d["C"])

    n = len(gemms)
    b2b_sp = timer.stats(lambda i: sparse(gemms[i % n]), n * passes, n)
    b2b_de = timer.stats(lambda i: dense(gemms[i % n]), n * passes, n)
    by_shape = {}
    for j, d in enumerate(gemms):
        ts = timer(lambda i, d=d: sparse(d), steps_gemm, 3)
        td = timer(lambda i, d=d: dense(d), steps_gemm, 3)
        e = by_shape.setdefault(d["shape"], dict(sparse_ms=0.0, dense_ms=0.0, count=0))
        e["sparse_ms"] += ts
        e["dense_ms"] += td
        e["count"] += 1
        if (j + 1) % 32 == 0:
            log(f"ViT-Large {dtype} stack: {j + 1} GEMMs timed one by one")
    flops = sum(2.0 * d["M"] * d["N"] * d["K"] for d in gemms)
    t_b2b, t_b2b_de = b2b_sp["ms"] * n, b2b_de["ms"] * n
    t_sum = sum(e["sparse_ms"] for e in by_shape.values())
    t_sum_de = sum(e["dense_ms"] for e in by_shape.values())
    unit = "tflops" if dtype == "f16" else "tops"
    del gemms, outs
    torch.cuda.empty_cache()
    return dict(workload=f"vit_large_stack_w24_{dtype}", gemms=n, layers=layers,
                t_back_to_back_ms=t_b2b, t_back_to_back_p10_ms=b2b_sp["p10"] * n,
                t_back_to_back_p90_ms=b2b_sp["p90"] * n, t_dense_back_to_back_ms=t_b2b_de,
                speedup_vs_dense_back_to_back=t_b2b_de / t_b2b,
                t_sum_per_gemm_ms=t_sum, t_dense_sum_per_gemm_ms=t_sum_de, speedup_vs_dense_sum=t_sum_de / t_sum,
                **{f"{unit}_dense_eq_back_to_back": flops / t_b2b / 1e9,
                   f"{unit}_nonzero_back_to_back": flops / 2 / t_b2b / 1e9},
                by_shape=by_shape)


def critical_density(sweep):
    """Density at which a pattern's kernel matches the dense kernel: linear
    interpolation between the two measured densities where the speedup
    crosses 1 (sweep: (density, speedup) ascending in density), or None."""
    crit = None
    for (d0, s0), (d1, s1) in zip(sweep, sweep[1:]):
        if s0 >= 1.0 > s1:
            crit = d0 + (s0 - 1.0) * (d1 - d0) / (s0 - s1)
    return crit


def patterns(torch, ssg, perf, wl, timer, steps, warmup, emit):
    """The pages' pattern comparison and critical-sparsity study (tile-wise
    slides: pattern-comparison and critical-sparsity tables) at the BERT-base
    FFN shape (M, K, N) = (4096, 768, 3072), fp16, one input set (cache-warm):
    dense; 2:4; tile-wise with G = 128 and G = 64 and block-wise with 64 x 64
    and 32 x 32 blocks (both run by the tile-wise kernel: a BW weight is a
    tile-wise weight, G = b, of whole b-row runs), each over a density sweep
    with the density where it matches dense; element-wise (unstructured)
    through torch's CSR sparse product in fp32, as the slides' cuSparse
    baseline ran in fp32.  Every pattern's first result is checked against
    the dense kernel on the same pruned weight (a tested kernel of this
    library) before it is timed."""
    rng = np.random.default_rng(0)
    M, K, N = 4096, 768, 3072
    A = wl.f16_normal(rng, (M, K))
    W = wl.f16_normal(rng, (K, N), 0.02)
    dev = torch.device("cuda")
    A_d = torch.from_numpy(A).to(dev)
    At = ssg.ssg_transpose_f16(A_d)
    C = torch.empty((M, N), dtype=torch.float16, device=dev)
    Wt = torch.from_numpy(np.ascontiguousarray(W.T)).to(dev)
    t_dense = timer(lambda i: ssg.dense_gemm_f16(A_d, Wt, out=C), steps, warmup)
    base = dict(shape=[M, K, N], t_dense_ms=t_dense, inputs="one set (cache-warm)")

    def dense_ref(Wp):
        """The dense kernel on the pruned weight, in float32."""
        Wpt = torch.from_numpy(np.ascontiguousarray(Wp.T)).to(dev)
        return ssg.dense_gemm_f16(A_d, Wpt).float()

    def rel_err(got, ref):
        return float((got.float() - ref).abs().max() / ref.abs().max().clamp_min(1e-30))

    Wp24 = wl.prune24_magnitude(W)
    vals, meta = ssg.w24_pack_f16(Wp24)
    v_d, m_d = torch.from_numpy(vals).to(dev), torch.from_numpy(meta.view(np.int32)).to(dev)
    err = rel_err(ssg.w24_gemm_f16(A_d, v_d, m_d), dense_ref(Wp24))
    t = timer(lambda i: ssg.w24_gemm_f16(A_d, v_d, m_d, out=C), steps, warmup)
    emit(dict(workload="patterns_2to4", density=0.5, t_ms=t, speedup_vs_dense=t_dense / t, check_rel_err=err,
              **base))
    fams = [("tilewise_g128", 128, lambda d: wl.prune_tilewise(W, 128, d), [0.1 * i for i in range(1, 10)]),
            ("tilewise_g64", 64, lambda d: wl.prune_tilewise(W, 64, d), [0.1 * i for i in range(1, 10)]),
            ("blockwise_64x64", 64, lambda d: wl.prune_blockwise(W, 64, d), [i / 12 for i in range(1, 12)]),
            ("blockwise_32x32", 32, lambda d: wl.prune_blockwise(W, 32, d), [i / 12 for i in range(1, 12)])]
    for name, G, prune, dens in fams:
        sweep = []
        for d in dens:
            Wp = prune(d)
            pk = ssg.tw_pack_f16(Wp, G).to(dev)
            err = rel_err(ssg.tw_gemm_f16(At, pk), dense_ref(Wp))
            if not err <= 1e-2:
                raise RuntimeError(f"{name} d={d}: result differs from the dense kernel (rel err {err:.3g})")
            t = timer(lambda i: ssg.tw_gemm_f16(At, pk, out=C), steps, warmup)
            dens_eff = float(np.count_nonzero(Wp)) / Wp.size
            sweep.append((dens_eff, t_dense / t))
            emit(dict(workload=f"patterns_{name}", density=d, density_nonzero=dens_eff, t_ms=t,
                      speedup_vs_dense=t_dense / t, check_rel_err=err, **base))
        crit = critical_density(sweep)
        emit(dict(workload=f"patterns_{name}_critical", critical_density=crit,
                  critical_sparsity=None if crit is None else 1.0 - crit,
                  note="nonzero density at which the pattern's kernel matches the dense kernel (linear "
                       "interpolation over the sweep)", **base))
    A32 = A_d.float()
    At32 = A32.t().contiguous()
    W32 = torch.from_numpy(W.astype(np.float32)).to(dev)
    t_dense32 = Timer(torch, graph=False)(lambda i: torch.matmul(A32, W32), steps, warmup)
    sweep = []
    for d in (0.01, 0.05, 0.2, 0.37, 0.5):
        Wp = wl.prune_elementwise(W, d)
        S = torch.from_numpy(np.ascontiguousarray(Wp.T.astype(np.float32))).to(dev).to_sparse_csr()
        try:
            got = torch.sparse.mm(S, At32).t()
            err = rel_err(got, dense_ref(Wp))
            if not err <= 1e-2:
                raise RuntimeError(f"element-wise d={d}: CSR result differs from the dense kernel "
                                   f"(rel err {err:.3g})")
            t = Timer(torch, graph=False)(lambda i: torch.sparse.mm(S, At32), steps, warmup)
            sweep.append((d, t_dense / t))
            emit(dict(workload="patterns_elementwise_csr_fp32", density=d, t_ms=t, check_rel_err=err,
                      speedup_vs_dense=t_dense / t, speedup_vs_dense_fp32=t_dense32 / t, t_dense_fp32_ms=t_dense32,
                      timing="eager (library call)", **base))
        except (RuntimeError, NotImplementedError) as e:
            emit(dict(workload="patterns_elementwise_csr_fp32", density=d, error=str(e)[:200], **base))
    crit = critical_density(sweep)
    emit(dict(workload="patterns_elementwise_csr_fp32_critical", critical_density=crit,
              critical_sparsity=None if crit is None else 1.0 - crit,
              note="None: slower than the dense kernel at every density measured" if crit is None else "",
              **base))


WORKLOADS = ("small", "vit_base_fc1", "bert_base_fc1", "bert_large_ffn", "vit_large", "vit_large_stack",
             "bert_base_fc1_i8", "patterns", "vit_large_shard8")
# table-mode selectors beside WORKLOADS: one GEMM of a workload (for profiling one kernel launch shape)
SUB_WORKLOADS = ("bert_large_fc1", "bert_large_fc2", "vit_large:qkv", "vit_large:proj", "vit_large:fc1",
                 "vit_large:fc2")


def table(a, torch, ssg, perf, wl, timer):
    rotate = not a.warm
    steps, warmup = a.steps, a.warmup
    want = set(a.workloads.split(",")) if a.workloads else set(WORKLOADS)
    timer.reps = 5
    timer.warm_s = TABLE_WARM_S

    vendor = not a.no_vendor

    peak = mfma_peak_measured(torch)
    if peak:
        print(json.dumps(dict(workload="mfma_peak_measured", **peak)), flush=True)

    def emit(d):
        if "t_vendor_sparse_ms" in d:
            d["speedup_vs_vendor_sparse"] = d["t_vendor_sparse_ms"] / d["t_sparse_ms"]
        f = measured_mfma_frac(d, peak)
        if f is not None:
            d["mfma_frac_of_measured_peak"] = f
        print(json.dumps(d), flush=True)

    if "small" in want:
        c = wl.make_small_w24_f16()
        r = w24_f16_case(torch, ssg, perf, c, steps, warmup, timer, rotate, vendor=vendor)
        nz, de = perf.w24_ops(c["M"], c["N"], c["K"])
        emit(dict(workload=c["name"] + "_w24_f16", shape=[c["M"], c["K"], c["N"]], **r,
                  tflops_nonzero=nz / r["t_sparse_ms"] / 1e9, tflops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                  speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                  speedup_vs_best_dense=min(r["t_dense_ms"], r["t_torch_ms"]) / r["t_sparse_ms"],
                  **perf.bound_report(nz, perf.w24_bytes(c["M"], c["N"], c["K"], 2, 2, 2), r["t_sparse_ms"],
                                      perf.PEAK_F16_TFLOPS * 1e12)))
    if "vit_base_fc1" in want:
        c = wl.make_vit_base_fc1_i8()
        r = w24_i8_case(torch, ssg, perf, c, steps, warmup, timer, rotate, with_f16_dense=True)
        r.pop("sets"), r.pop("sp")
        nz, de = perf.w24_ops(c["M"], c["N"], c["K"])
        b = perf.w24_bytes(c["M"], c["N"], c["K"], 1, 1, 4, True)
        emit(dict(workload=c["name"] + "_w24_i8", shape=[c["M"], c["K"], c["N"]], **r,
                  tops_nonzero=nz / r["t_sparse_ms"] / 1e9, tops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                  gbs=b / r["t_sparse_ms"] / 1e6, speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                  speedup_vs_dense_f16=r["t_dense_f16_ms"] / r["t_sparse_ms"],
                  **perf.bound_report(nz, b, r["t_sparse_ms"], perf.PEAK_I8_TOPS * 1e12)))
        torch.cuda.empty_cache()
        for out_type in ("f16", "i8"):
            r = w24_i8_out_case(torch, ssg, perf, c, out_type, steps, warmup, timer, rotate, vendor=vendor)
            b = perf.w24_bytes(c["M"], c["N"], c["K"], 1, 1, r["out_bytes"], True)
            emit(dict(workload=f"vit_base_fc1_w24_i8_{out_type}_out", shape=[c["M"], c["K"], c["N"]], **r,
                      tops_nonzero=nz / r["t_sparse_ms"] / 1e9, tops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                      gbs=b / r["t_sparse_ms"] / 1e6, speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                      **perf.bound_report(nz, b, r["t_sparse_ms"], perf.PEAK_I8_TOPS * 1e12)))
            torch.cuda.empty_cache()
    tw_cases = []
    if "bert_base_fc1" in want:
        tw_cases.append(wl.make_bert_base_fc1_tw())
    if want & {"bert_large_ffn", "bert_large_fc1", "bert_large_fc2"}:
        c4 = wl.make_bert_large_ffn_tw()
        tw_cases += [c4[g] for g in ("fc1", "fc2") if want & {"bert_large_ffn", "bert_large_" + g}]
    for c in tw_cases:
        r = tw_case(torch, ssg, perf, c, steps, warmup, timer, rotate, extras=not a.no_tw_extras)
        emit(dict(workload=c["name"] + "_tw_f16", shape=[c["M"], c["K"], c["N"]], **r,
                  tflops_nonzero=r["ops"] / r["t_sparse_ms"] / 1e9, gbs=r["bytes"] / r["t_sparse_ms"] / 1e6,
                  speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                  speedup_vs_best_dense=min(r["t_dense_ms"], r["t_torch_ms"]) / r["t_sparse_ms"],
                  speedup_vs_dense_incl_transpose=r["t_dense_ms"] / (r["t_sparse_ms"] + r["t_transpose_ms"]),
                  **perf.bound_report(r["ops"], r["bytes"], r["t_sparse_ms"], perf.PEAK_F16_TFLOPS * 1e12)))
        torch.cuda.empty_cache()
    if "patterns" in want:
        patterns(torch, ssg, perf, wl, timer, steps, warmup, emit)
        torch.cuda.empty_cache()
    if "bert_base_fc1_i8" in want:
        c = wl.make_bert_base_fc1_tw_i8()
        for out_type in ("f16", "i8"):
            r = tw_i8_case(torch, ssg, perf, c, out_type, steps, warmup, timer, rotate)
            emit(dict(workload=f"bert_base_fc1_tw_i8_{out_type}_out", shape=[c["M"], c["K"], c["N"]], **r,
                      tops_nonzero=r["ops"] / r["t_sparse_ms"] / 1e9,
                      speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"]))
            torch.cuda.empty_cache()
    only5 = {w.split(":", 1)[1] for w in want if w.startswith("vit_large:")}
    if "vit_large" in want or only5:
        for g in wl.vit_large_layers("f16", layers=1):
            if only5 and g["name"].rsplit("_", 1)[1] not in only5:
                continue
            r = w24_f16_case(torch, ssg, perf, g, steps, warmup, timer, rotate, vendor=vendor)
            nz, de = perf.w24_ops(g["M"], g["N"], g["K"])
            emit(dict(workload=g["name"] + "_w24_f16", shape=[g["M"], g["K"], g["N"]], **r,
                      tflops_nonzero=nz / r["t_sparse_ms"] / 1e9, tflops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                      speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                      speedup_vs_best_dense=min(r["t_dense_ms"], r["t_torch_ms"]) / r["t_sparse_ms"],
                      **perf.bound_report(nz, perf.w24_bytes(g["M"], g["N"], g["K"], 2, 2, 2), r["t_sparse_ms"],
                                          perf.PEAK_F16_TFLOPS * 1e12)))
            torch.cuda.empty_cache()
    if "vit_large_shard8" in want:
        # one GPU's share of the ViT-L layer when the 4096 tokens are split over
        # 8 GPUs (M = 512 rows each; the packed weights are replicated)
        M8 = wl.VIT_LARGE_M // 8
        for g in wl.vit_large_layers("f16", layers=1, M=M8):
            r = w24_f16_case(torch, ssg, perf, g, steps, warmup, timer, rotate, vendor=vendor)
            nz, de = perf.w24_ops(g["M"], g["N"], g["K"])
            emit(dict(workload=g["name"].replace("vit_large_", "vit_large_shard8_") + "_w24_f16",
                      shape=[g["M"], g["K"], g["N"]], **r,
                      tflops_nonzero=nz / r["t_sparse_ms"] / 1e9, tflops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                      speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                      speedup_vs_best_dense=min(r["t_dense_ms"], r["t_torch_ms"]) / r["t_sparse_ms"],
                      **perf.bound_report(nz, perf.w24_bytes(g["M"], g["N"], g["K"], 2, 2, 2), r["t_sparse_ms"],
                                          perf.PEAK_F16_TFLOPS * 1e12)))
            torch.cuda.empty_cache()
        for g in wl.vit_large_layers("i8", layers=1, M=M8):
            r = w24_i8_case(torch, ssg, perf, g, steps, warmup, timer, rotate)
            r.pop("sets"), r.pop("sp")
            nz, de = perf.w24_ops(g["M"], g["N"], g["K"])
            b = perf.w24_bytes(g["M"], g["N"], g["K"], 1, 1, 4, True)
            emit(dict(workload=g["name"].replace("vit_large_", "vit_large_shard8_") + "_w24_i8",
                      shape=[g["M"], g["K"], g["N"]], **r,
                      tops_nonzero=nz / r["t_sparse_ms"] / 1e9, tops_dense_eq=de / r["t_sparse_ms"] / 1e9,
                      speedup_vs_dense=r["t_dense_ms"] / r["t_sparse_ms"],
                      **perf.bound_report(nz, b, r["t_sparse_ms"], perf.PEAK_I8_TOPS * 1e12)))
            torch.cuda.empty_cache()
    if "vit_large_stack" in want:
        f16 = vit_large_stack(torch, ssg, perf, wl, "f16", timer)
        emit(f16)
        i8 = vit_large_stack(torch, ssg, perf, wl, "i8", timer)
        # int8 against the fp16 dense stack of the same shapes as well
        i8["t_dense_f16_back_to_back_ms"] = f16["t_dense_back_to_back_ms"]
        i8["speedup_vs_dense_f16_back_to_back"] = f16["t_dense_back_to_back_ms"] / i8["t_back_to_back_ms"]
        emit(i8)
    return 0


if __name__ == "__main__":
    sys.exit(main())
