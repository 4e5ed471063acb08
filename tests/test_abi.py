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
        m = re.match(r"^\s*(?:int|const char \*)\s*(\w+)\s*\(", line)
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
    (lambda r: r.tw_gemm_f16_ex(*[_p(16)] * 8, 2, 16, 0, 2, 4, _p(16), 8, 32, 64, None), "unknown flags"),
    (lambda r: r.tw_gemm_i8(*[_p(16)] * 8, 2, 16, _p(16), None, _p(16), 2, 24, 32, 64, None), "multiple of 16"),
    (lambda r: r.tw_gemm_i8(*[_p(16)] * 8, 2, 16, None, None, _p(16), 2, 32, 32, 64, None), "needs scale"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 24, _p(16), 8, 48, 64, None), "G=24"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 256, _p(16), 8, 512, 64, None), "at most 128"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 3, 16, _p(16), 8, 32, 64, None), "T=3"),
    (lambda r: r.tw_gemm_f16(*[_p(16)] * 8, 2, 16, _p(16), 12, 32, 64, None), "multiple of 8"),
    (lambda r: r.ssg_transpose_f16(_p(16), _p(16), 12, 16, None), "multiples of 8"),
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
