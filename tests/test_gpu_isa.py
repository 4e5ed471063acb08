"""Operand / index / accumulator layouts of the gfx950 matrix instructions that
the kernels rely on, checked on one wave with small exact integers.

The 2:4 kernels assume (h = lane / 32, r = lane % 32):
  sparse operand   lane holds the kept values of row r for k in [16h, 16h+16)
                   (f16) or [32h, 32h+32) (i8), two per group of four, with
                   slot c's 2-bit position at bits 2c of the index operand;
  dense operand    lane holds two runs of column r: elements 0..7 are
                   k = 8h .. 8h+7 and elements 8..15 are k = 16+8h .. (f16);
                   for i8 the runs are 16 long (k = 16h .., k = 32+16h ..);
  accumulator      register i of lane l is D[8*(i/4) + 4h + i%4][r].
The dense kernels only need that element e of a lane's row operand and of its
column operand refer to the same k, plus the accumulator layout.

On a mismatch the test writes basis experiments (one 1 in the sparse operand,
distinct ids in the dense operand) to the directory named by SSG_PROBE_DUMP (or
the system temporary directory) for offline decoding.
"""

import ctypes as ct
import os
import tempfile

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "tests", "probes", "libssg_probe.so")

# op: (A elems/lane, B elems/lane, D regs/lane, numpy dtype, acc dtype)
OPS = {
    0: (8, 16, 16, np.float16, np.float32),   # smfmac f32 32x32x32 f16
    1: (16, 32, 16, np.int8, np.int32),       # smfmac i32 32x32x64 i8
    2: (8, 8, 16, np.float16, np.float32),    # mfma f32 32x32x16 f16
    3: (8, 8, 4, np.float16, np.float32),     # mfma f32 16x16x32 f16
    4: (16, 16, 16, np.int8, np.int32),       # mfma i32 32x32x32 i8
}
PAIRS = [(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)]


@pytest.fixture(scope="module")
def probe(gpu):
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} missing: run __graft_entry__.build()")
    lib = ct.CDLL(PROBE)
    lib.probe_run.argtypes = [ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p, ct.c_void_p]
    lib.probe_run.restype = ct.c_int
    return lib


def run(probe, op, a, b, idx):
    import torch
    na, nb, nd, dt, acc = OPS[op]
    E = a.shape[0]
    ta = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tb = torch.from_numpy(np.ascontiguousarray(b)).cuda()
    ti = torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).cuda()
    td = torch.empty((E, 64, nd), dtype=torch.float32 if acc == np.float32 else torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = probe.probe_run(op, E, ta.data_ptr(), tb.data_ptr(), ti.data_ptr(), td.data_ptr(), stream)
    assert rc == 0, f"probe_run returned {rc}"
    return td.cpu().numpy()


def model(op, a, b, idx):
    """Expected lane outputs under the assumed layouts (one experiment)."""
    na, nb, nd, dt, acc = OPS[op]
    a = a.astype(np.int64) if dt == np.int8 else a.astype(np.float64)
    b = b.astype(np.int64) if dt == np.int8 else b.astype(np.float64)
    if op == 3:
        Am = np.zeros((16, 32), a.dtype)
        Bm = np.zeros((32, 16), b.dtype)
        for l in range(64):
            q = l // 16
            Am[l % 16, q * 8:q * 8 + 8] = a[l]
            Bm[q * 8:q * 8 + 8, l % 16] = b[l]
        D = Am @ Bm
        return np.array([[D[(l // 16) * 4 + i, l % 16] for i in range(4)] for l in range(64)])
    span = {0: 32, 1: 64, 2: 16, 4: 32}[op]
    Am = np.zeros((32, span), a.dtype)
    Bm = np.zeros((span, 32), b.dtype)
    for l in range(64):
        h, r = l // 32, l % 32
        if op in (0, 1):
            for c in range(na):
                pos = (int(idx[l]) >> (2 * c)) & 3
                Am[r, h * (span // 2) + (c // 2) * 4 + pos] += a[l, c]
        else:
            Am[r, h * (span // 2):(h + 1) * (span // 2)] = a[l]
        if op in (0, 1):
            run = nb // 2
            for e in range(nb):
                Bm[2 * run * (e // run) + run * h + e % run, r] = b[l, e]
        else:
            Bm[h * (span // 2):(h + 1) * (span // 2), r] = b[l]
    D = Am @ Bm
    return np.array([[D[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] for i in range(16)] for l in range(64)])


def random_idx(rng, groups):
    words = np.zeros(64, np.int64)
    for l in range(64):
        w = 0
        for g in range(groups):
            p0, p1 = PAIRS[rng.integers(0, 6)]
            w |= (p0 | p1 << 2) << (4 * g)
        words[l] = w
    return words.astype(np.uint32).view(np.int32)


def dump_discovery(probe, op):
    """Basis experiments for decoding the sparse layouts offline."""
    na, nb, nd, dt, acc = OPS[op]
    E = 64 * na
    a = np.zeros((E, 64, na), dt)
    for e in range(E):
        a[e, e // na, e % na] = 1
    ids = (np.arange(64 * nb) % (127 if dt == np.int8 else 2048)).reshape(64, nb).astype(dt)
    b = np.broadcast_to(ids, (E, 64, nb)).copy()
    fixed = np.full((E, 64), 0x44444444, np.uint32).view(np.int32)
    d_fixed = run(probe, op, a, b, fixed)
    rng = np.random.default_rng(99)
    ridx = np.stack([random_idx(rng, na // 2) for _ in range(E)])
    d_rand = run(probe, op, a, b, ridx)
    out = os.environ.get("SSG_PROBE_DUMP") or tempfile.gettempdir()
    os.makedirs(out, exist_ok=True)
    path = os.path.join(out, f"isa_discovery_op{op}.npz")
    np.savez(path, a=a, b=b, idx_fixed=fixed, d_fixed=d_fixed, idx_rand=ridx, d_rand=d_rand)
    return path


@pytest.mark.parametrize("op", [0, 1, 2, 3, 4])
def test_instruction_layout(probe, op):
    na, nb, nd, dt, acc = OPS[op]
    rng = np.random.default_rng(op)
    E = 8
    a = rng.integers(-3, 4, size=(E, 64, na)).astype(dt)
    b = rng.integers(-3, 4, size=(E, 64, nb)).astype(dt)
    idx = np.stack([random_idx(rng, max(1, na // 2)) for _ in range(E)]) if op in (0, 1) \
        else np.zeros((E, 64), np.int32)
    d = run(probe, op, a, b, idx)
    ok = all(np.array_equal(d[e].astype(np.float64), model(op, a[e], b[e], idx[e]).astype(np.float64))
             for e in range(E))
    if not ok:
        path = dump_discovery(probe, op) if op in (0, 1) else "n/a"
        pytest.fail(f"op {op}: layout differs from the kernels' assumption; discovery data: {path}")
