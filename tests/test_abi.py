"""The C-ABI library loads without a GPU, exports every symbol its header
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes as ct
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssg.h")


def declared_functions():
    names = []
    for line in open(HEADER):
        m = re.match(r"^\s*(?:int|int32_t|int64_t|const char \*)\s*(\w+)\s*\(", line)
        if m:
            names.append(m.group(1))
    return names


def test_header_declares_the_path():
    names = set(declared_functions())
    assert {"w24_pack_f16", "w24_pack_i8", "w24_unpack_f16", "w24_unpack_i8", "tw_pack_query",
            "tw_pack_f16", "tw_unpack_f16", "dense_gemm_f16", "dense_gemm_i8", "w24_gemm_f16",
            "w24_gemm_i8", "tw_gemm_f16", "ssg_transpose_f16", "ssg_last_error",
            "dense_gemm_i8_out", "w24_gemm_i8_out", "tw_gemm_f16_ex", "tw_pack_i8", "tw_unpack_i8",
            "tw_pack_query_i8", "tw_gemm_i8"} <= names


def test_every_declared_symbol_is_exported(lib):
    raw = lib.load()
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_only_declared_symbols_are_exported(lib):
    out = os.popen(f"nm -D --defined-only {lib.lib_path()}").read().split("\n")
    exported = {l.split()[-1] for l in out if " T " in l}
    assert exported <= set(declared_functions()), exported - set(declared_functions())


def test_version(lib):
    assert lib.load().ssg_version().decode().startswith("ssg ")


def _raw(lib):
    return lib.load()


def _p(v):
    return ct.c_void_p(v)


def has_device(lib):
    buf = ct.create_string_buffer(64)
    return _raw(lib).ssg_device_arch(buf, 64) == 0


@pytest.mark.parametrize("call,msg", [
    (lambda r: r.dense_gemm_f16(_p(16), _p(16), _p(16), 8, 64, 100, None), "multiple of 64"),
    (lambda r: r.dense_gemm_f16(_p(16), _p(16), _p(16), -1, 64, 64, None), "M=-1"),
    (lambda r: r.dense_gemm_i8(_p(16), _p(16), None, _p(16), 8, 64, 64, None), "multiple of 128"),
    (lambda r: r.w24_gemm_f16(None, _p(16), _p(16), _p(16), 8, 64, 64, None), "null"),
    (lambda r: r.w24_gemm_f16(_p(18), _p(16), _p(16), _p(16), 8, 64, 64, None), "aligned"),
    (lambda r: r.w24_gemm_f16(_p(16), _p(16), None, _p(16), 8, 64, 64, None), "meta"),
    (lambda r: r.w24_gemm_i8(_p(16), _p(16), _p(16), _p(20), _p(16), 8, 64, 128, None), "scale"),
    (lambda r: r.w24_gemm_i8(_p(16), _p(16), _p(16), None, _p(16), 8, 96, 128, None), "multiple of 64"),
    (lambda r: r.w24_gemm_i8_out(*[_p(16)] * 5, _p(16), 7, 8, 64, 128, None), "unknown out_type"),
    (lambda r: r.w24_gemm_i8_out(*[_p(16)] * 5, _p(16), 0, 8, 64, 128, None), "no scale or bias"),
    (lambda r: r.w24_gemm_i8_out(*[_p(16)] * 3, None, None, _p(16), 2, 8, 64, 128, None), "needs scale"),
    (lambda r: r.dense_gemm_i8_out(*[_p(16)] * 3, _p(36), _p(16), 3, 8, 64, 128, None), "16-byte aligned"),
    (lambda r: r.dense_gemm_i8_out(*[_p(16)] * 4, _p(16), 1, 8, 64, 100, None), "multiple of 128"),
    (lambda r: r.tw_gemm_f16_ex(*[_p(16)] * 8, 2, 16, 1, 2, 0, _p(16), 8, 32, 64, None), "tile range"),
    (lambda r: r.tw_gemm_f16_ex(*[_p(16)] * 8, 2, 16, 0, 0, 0, _p(16), 8, 32, 64, None), "tile range"),
    (lambda r: r.tw_gemm_f16_ex(*[_p(16)] * 8, 2, 16, 0, 2, 8, _p(16), 8, 32, 64, None), "unknown flags"),
    (lambda r: r.tw_gemm_f16_ex(*[_p(16)] * 8, 2, 16, 0, 2, 4 | 16, _p(16), 8, 32, 64, None), "unknown flags"),
    (lambda r: r.tw_gemm_i8(*[_p(16)] * 8, 2, 272, _p(16), None, _p(16), 2, 24, 544, 64, None), "at most 256"),
    (lambda r: r.tw_gemm_i8(*[_p(16)] * 8, 2, 16, None, None, _p(16), 2, 32, 32, 64, None), "needs scale"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 24, _p(16), 8, 48, 64, None), "G=24"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 272, _p(16), 8, 544, 64, None), "at most 256"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 3, 16, _p(16), 8, 32, 64, None), "T=3"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 16, _p(16), -3, 32, 64, None), "bad shape"),
    (lambda r: r.w24_gemm_f16_splitk_static(*[_p(16)] * 4, 4096, 1024, 4096, 8, None), "static scratch"),
    (lambda r: r.w24_gemm_f16_splitk_static(*[_p(16)] * 4, 8, 64, 128, 3, None), "splits=3"),
    (lambda r: r.w24_gemm_f16_splitk_static(*[_p(16)] * 4, 8, 64, 128, 0, None), "splits=0"),
    (lambda r: r.ssg_transpose_f16(_p(16), _p(16), 12, 16, None), "multiples of 8"),
    (lambda r: r.w24_gemm_f16_splitk(*[_p(16)] * 4, 8, 64, 128, 3, _p(16), 1 << 20, None), "splits=3"),
    (lambda r: r.w24_gemm_f16_splitk(*[_p(16)] * 4, 8, 64, 128, 0, _p(16), 1 << 20, None), "splits=0"),
    (lambda r: r.dense_gemm_f16_splitk(*[_p(16)] * 3, 8, 64, 128, 128, _p(16), 1 << 20, None), "splits=128"),
    (lambda r: r.w24_gemm_f16_splitk(*[_p(16)] * 4, 8, 64, 128, 2, None, 1 << 20, None), "workspace null"),
    (lambda r: r.w24_gemm_f16_splitk(*[_p(16)] * 4, 8, 64, 128, 2, _p(20), 1 << 20, None), "16-byte aligned"),
    (lambda r: r.w24_gemm_f16_splitk(*[_p(16)] * 4, 8, 64, 128, 2, _p(16), 4095, None), "4096 needed"),
    (lambda r: r.w24_gemm_i8_splitk(*[_p(16)] * 5, _p(16), 9, 8, 64, 256, 2, _p(16), 1 << 20, None),
     "unknown out_type"),
    (lambda r: r.dense_gemm_i8_splitk(*[_p(16)] * 2, None, None, _p(16), 1, 8, 64, 256, 2, _p(16), 1 << 20, None),
     "needs scale"),
    (lambda r: r.w24_gemm_i8_splitk(*[_p(16)] * 5, _p(16), 1, 8, 64, 256, 4, _p(16), 1 << 20, None), "splits=4"),
    (lambda r: r.w24_gemm_i8_splitk(_p(16), _p(16), None, _p(16), None, _p(16), 1, 8, 64, 256, 2, _p(16), 1 << 20,
                                    None), "meta"),
])
def test_invalid_arguments_rejected_on_host(lib, call, msg):
    raw = _raw(lib)
    assert call(raw) == 1  # SSG_EINVAL
    assert msg in raw.ssg_last_error().decode()


def test_zero_rows_is_ok_without_touching_the_device(lib):
    raw = _raw(lib)
    assert raw.w24_gemm_f16(None, None, None, None, 0, 64, 64, None) == 0
    assert raw.tw_gemm_f16(*[None] * 8, 2, 16, None, 0, 32, 64, None) == 0


def test_valid_arguments_without_gpu_give_enodev(lib):
    if has_device(lib):
        pytest.skip("a device is present: this checks the no-device path only")
    raw = _raw(lib)
    assert raw.w24_gemm_f16(_p(16), _p(16), _p(16), _p(16), 8, 64, 64, None) == 4  # SSG_ENODEV
    assert "no HIP device" in raw.ssg_last_error().decode()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import structured_sparse_gemm_w24_amd._lib as L
    monkeypatch.setenv("SSG_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(L, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        L.w24_pack_f16(np.zeros((4, 1), np.float16))


def test_concurrent_packs_and_thread_local_errors(lib):
    """Host calls are re-entrant: packs from several threads at once give the
    sequential results, and each thread's ssg_last_error() reports its own
    call (a failing pack on one thread does not overwrite another's message)."""
    import threading

    import workloads as wl

    raw = lib.load()
    cases = [wl.random_24_i8(np.random.default_rng(s), 1, 256, 192)["Wp"] for s in range(8)]
    want = [lib.w24_pack_i8(W) for W in cases]
    got = [None] * len(cases)
    errors = [None] * len(cases)
    bad = np.ones((8, 64), np.int8)  # four nonzeros per group: not 2:4

    def work(i):
        for _ in range(20):
            got[i] = lib.w24_pack_i8(cases[i])
            if i % 2:
                vals = np.empty((64, 4), np.int8)
                meta = np.empty((64, 1), np.uint32)
                rc = raw.w24_pack_i8(bad.ctypes.data_as(ct.c_void_p), 8, 64, vals.ctypes.data_as(ct.c_void_p),
                                     meta.ctypes.data_as(ct.c_void_p))
                errors[i] = (rc, raw.ssg_last_error().decode())
            else:
                rc = raw.ssg_version()
                errors[i] = (0, raw.ssg_last_error().decode())

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i in range(len(cases)):
        assert np.array_equal(got[i][0], want[i][0]) and np.array_equal(got[i][1], want[i][1])
        rc, msg = errors[i]
        if i % 2:
            assert rc == 2 and "nonzeros" in msg
        else:
            assert msg == ""  # the last call on this thread (a successful pack) cleared it


def test_splitk_host_helpers(lib):
    raw = _raw(lib)
    assert raw.ssg_splitk_workspace_bytes(512, 1024, 8) == 8 * 512 * 1024 * 4
    assert raw.ssg_splitk_workspace_bytes(512, 1024, 1) == 0
    assert raw.ssg_splitk_workspace_bytes(-1, 1024, 8) == 0
    # one GPU's share of ViT-L fc2 (M = 512): fp16 has 64 K stages -> split, on
    # 128 x 128 tiles x 8 (256 workgroups); int8 32 -> none; int8 at K = 8192 -> split
    assert lib.splitk_suggest(lib.SSG_KIND_W24_F16, 512, 1024, 4096) == 8
    assert lib.splitk_suggest(lib.SSG_KIND_W24_I8, 512, 1024, 4096) == 1
    assert lib.splitk_suggest(lib.SSG_KIND_W24_I8, 512, 1024, 8192) == 2
    # 128 x 4096 output: 32 tiles of 128 x 128 x 8 splits
    assert lib.splitk_suggest(lib.SSG_KIND_W24_F16, 128, 4096, 4096) == 8
    # 256 x 1024: 128 x 128 x 8 and 64 x 128 x 4 stay under 256 workgroups ->
    # 64 x 64 tiles (64 of them) x 4
    assert lib.splitk_suggest(lib.SSG_KIND_W24_F16, 256, 1024, 4096) == 4
    # more than 128 tiles -> no split (1024 x 1024 output: 256 tiles of 64 x 64)
    assert lib.splitk_suggest(lib.SSG_KIND_W24_F16, 1024, 1024, 4096) == 1
    # the ViT-Base fc1 shape fills the chip several times over -> no split
    for kind in range(4):
        assert lib.splitk_suggest(kind, 12608, 3072, 768) == 1
    # every suggestion divides the K stages and leaves >= 8 per split
    for kind in range(4):
        for M, N, K in ((512, 1024, 4096), (512, 3072, 1024), (64, 256, 8192), (1, 64, 2048)):
            p = lib.splitk_suggest(kind, M, N, K)
            stages = K // (128 if kind >= 2 else 64)
            assert p >= 1 and stages % p == 0 and (p == 1 or stages // p >= 8), (kind, M, N, K, p)
    assert lib.splitk_suggest(7, 512, 1024, 4096) == 1
    assert lib.splitk_suggest(1, 0, 1024, 4096) == 1


def test_tile_choice_host_query(lib):
    F16, D16, I8, D8 = lib.SSG_KIND_W24_F16, lib.SSG_KIND_DENSE_F16, lib.SSG_KIND_W24_I8, lib.SSG_KIND_DENSE_I8
    # the headline shape (ViT-Base fc1, int8): 2376 tiles of 128 x 128
    assert lib.tile_choice(I8, 12608, 3072, 768) == (128, 128)
    assert lib.tile_choice(D8, 12608, 3072, 768) == (128, 128)
    # ViT-L fc1 (fp16): 256 x 256 tiles fill the chip
    assert lib.tile_choice(F16, 4096, 4096, 1024) == (256, 256)
    # one GPU's share of ViT-L (M = 512): proj on one-wave 32 x 32 tiles (512 of
    # them, 16 / 8 K stages), the wider layers on 64-row tiles
    for kind in (F16, D16, I8, D8):
        assert lib.tile_choice(kind, 512, 1024, 1024) == (32, 32)
        assert lib.tile_choice(kind, 520, 1024, 1024) == (64, 64)  # 544 tiles of 32 x 32
    # 64 or more K stages: 64 x 64 tiles (and split K) instead of 32 x 32
    assert lib.tile_choice(F16, 512, 1024, 4096) == (64, 64)
    assert lib.tile_choice(F16, 512, 1024, 4032) == (32, 32)
    assert lib.tile_choice(I8, 512, 1024, 4096) == (32, 32)  # 32 stages of 128
    assert lib.tile_choice(I8, 512, 1024, 8192) == (64, 64)
    assert lib.tile_choice(F16, 512, 4096, 1024) == (64, 128)  # 64 x 64 tiles would number 512
    assert lib.tile_choice(I8, 512, 4096, 1024) == (64, 64)
    # 192 tiles of 128 x 128: int8 at short K takes 64 x 64, fp16 and long-K int8 do not
    assert lib.tile_choice(I8, 1024, 3072, 1024) == (64, 64)
    assert lib.tile_choice(F16, 1024, 3072, 1024) == (128, 128)
    assert lib.tile_choice(I8, 1024, 3072, 4096) == (128, 128)
    assert lib.tile_choice(7, 512, 1024, 1024) == (0, 0)
    assert lib.tile_choice(F16, 0, 1024, 1024) == (0, 0)


def test_splitk_zero_rows_is_ok_without_touching_the_device(lib):
    raw = _raw(lib)
    assert raw.w24_gemm_f16_splitk(None, None, None, None, 0, 64, 128, 2, None, 0, None) == 0


def test_vendor_baseline_is_outside_the_product():
    """The bench's hipSPARSELt baseline lives in its own library: libssg does not
    link hipSPARSELt and the package never names the vendor library."""
    import glob
    import subprocess
    import structured_sparse_gemm_w24_amd as ssg
    pkg = os.path.dirname(ssg.__file__)
    dyn = subprocess.run(["readelf", "-d", os.path.join(pkg, "libssg.so")], capture_output=True, text=True)
    assert dyn.returncode == 0 and "NEEDED" in dyn.stdout
    assert "hipsparselt" not in dyn.stdout.lower()
    for path in glob.glob(os.path.join(pkg, "*.py")) + glob.glob(os.path.join(pkg, "csrc", "*.*")) + \
            glob.glob(os.path.join(pkg, "csrc", "kernels", "*.*")):
        if path.endswith("build.py"):
            continue  # the build step is what builds the separate bench library
        text = open(path, errors="replace").read()
        assert "libssg_vendor" not in text and "hipsparselt" not in text.lower(), path


def test_mfma_peak_probe_is_outside_the_product():
    """The bench's matrix-core rate probe is a separate library with one export;
    libssg neither exports it nor names the probe library."""
    import ctypes as ct
    import glob
    import subprocess
    import structured_sparse_gemm_w24_amd as ssg
    pkg = os.path.dirname(ssg.__file__)
    probe = os.path.join(pkg, "libssg_peak.so")
    assert os.path.exists(probe), "build() builds the probe beside libssg"
    syms = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True).stdout
    assert "ssg_bench_mfma_peak" in syms
    main = subprocess.run(["nm", "-D", "--defined-only", os.path.join(pkg, "libssg.so")],
                          capture_output=True, text=True).stdout
    assert "ssg_bench_mfma_peak" not in main
    for path in glob.glob(os.path.join(pkg, "*.py")) + glob.glob(os.path.join(pkg, "csrc", "*.*")) + \
            glob.glob(os.path.join(pkg, "csrc", "kernels", "*.*")):
        if path.endswith("build.py"):
            continue
        assert "libssg_peak" not in open(path, errors="replace").read(), path
    # invalid arguments are refused before any launch (no device needed for that)
    fn = ct.CDLL(probe).ssg_bench_mfma_peak
    fn.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]
    assert fn(4, 1, 1, None, None) != 0 and fn(0, 0, 1, None, None) != 0


def test_single_hip_runtime_after_load():
    """Loading the library (before anything touched torch) leaves one HIP
    runtime in the process: the binding imports torch first, so the library
    binds to the runtime torch carries instead of loading a second one."""
    import subprocess
    import sys
    code = ("import structured_sparse_gemm_w24_amd as s; s.load(); "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    libs = eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
