"""The bench's report arithmetic, pinned by the one detailed table on the pages
(tile-wise slides, BERT-Base 75 % time breakdown; see tests/golden)."""

import os

import pytest

from structured_sparse_gemm_w24_amd import perf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tw_bert_base_time_breakdown.txt")


def load_table():
    rows, printed = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) == 7:
            rows[parts[0]] = dict(gemm=float(parts[1]), non_gemm=float(parts[2]),
                                  transpose=float(parts[3]), total=float(parts[4]),
                                  speedup=float(parts[5]),
                                  share=None if parts[6] == "-" else float(parts[6]))
        else:
            printed[parts[0]] = float(parts[1])
    return rows, printed


def test_totals_add_up():
    rows, _ = load_table()
    for r in rows.values():
        assert r["gemm"] + r["non_gemm"] + r["transpose"] == pytest.approx(r["total"], abs=0.006)


def test_speedups_and_shares_reproduce_printed_values():
    rows, printed = load_table()
    base = rows["dense"]["total"]
    for name, r in rows.items():
        s = perf.speedup(base, r["total"])
        digits = len(str(r["speedup"]).split(".")[1]) if "." in str(r["speedup"]) else 0
        assert round(s, digits) == r["speedup"], name
        if r["share"] is not None:
            assert round(100 * perf.share(r["gemm"], r["total"])) == r["share"], name
    g = perf.speedup(rows["dense"]["gemm"], rows["fused_transpose"]["gemm"])
    assert round(g, 2) == pytest.approx(printed["gemm_speedup_vs_dense"], abs=0.011)
    g2 = perf.speedup(rows["without_transpose"]["gemm"], rows["fused_transpose"]["gemm"])
    assert round(g2, 2) == printed["gemm_speedup_vs_without_transpose"]


def test_work_models_closed_form():
    M, N, K = 12608, 3072, 768
    nz, de = perf.w24_ops(M, N, K)
    assert de == 2 * nz == 2 * M * N * K
    b = perf.w24_bytes(M, N, K, 1, 1, 4, scale=True)
    assert b == M * K + N * K // 2 + N * K // 8 + 4 * N + 4 * M * N
    assert perf.dense_bytes(4, 8, 16, 2, 2, 2) == 4 * 16 * 2 + 16 * 8 * 2 + 4 * 8 * 2
    assert perf.transpose_bytes(3, 5) == 60
    r = perf.roofline(4000.0, perf.PEAK_HBM_GBS, "GB/s", "hbm")
    assert r["frac"] == 0.5 and r["traffic"] is None


def test_bound_report_matches_the_closed_forms():
    # 2:4 int8 at 12608x768x3072 with fp32 output: 29.7 G nonzero ops at 5 POP/s
    # is 5.95 us, 166.1 MB at 8 TB/s is 20.76 us, so HBM binds
    nz, _ = perf.w24_ops(12608, 3072, 768)
    r = perf.bound_report(nz, perf.w24_bytes(12608, 3072, 768, 1, 1, 4, scale=True), 0.04152,
                          perf.PEAK_I8_TOPS * 1e12)
    assert r["bound"] == "hbm"
    assert abs(r["t_ideal_hbm_us"] - 20.762) < 0.01 and abs(r["t_ideal_mfma_us"] - 5.949) < 0.01
    assert abs(r["roofline_frac"] - 0.5) < 1e-3
    # 2:4 fp16 ViT-L qkv 4096x1024x3072: MFMA binds (5.15 us vs 4.64 us)
    nz, _ = perf.w24_ops(4096, 3072, 1024)
    r = perf.bound_report(nz, perf.w24_bytes(4096, 3072, 1024, 2, 2, 2), 0.0103, perf.PEAK_F16_TFLOPS * 1e12)
    assert r["bound"] == "mfma" and abs(r["roofline_frac"] - 0.5) < 1e-3


def test_gfx_clock_parser_reads_every_xcd_and_nothing_else():
    import bench
    doc = {"gpu_data": [{"gpu": 0, "clock": {
        **{f"gfx_{i}": {"clk": {"value": 1400 + 10 * i, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                        "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED"} for i in range(8)},
        "mem_0": {"clk": {"value": 1900, "unit": "MHz"}},
        "vclk_0": {"clk": {"value": 29, "unit": "MHz"}}}}]}
    assert bench._gfx_clocks(doc) == [1400.0 + 10 * i for i in range(8)]
    assert bench._gfx_clocks({"gpu_data": []}) == []


def test_kernel_hash_ignores_comments_and_layout():
    import bench
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n/* note */\n"
    b = "/* header\n   text */ int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)


def test_cpu_baseline_parity_field():
    """The headline's oracle leg compares a GPU output with the oracle bit for
    bit; a single changed element must flip the verdict."""
    import numpy as np

    import bench
    import oracle
    import workloads as wl
    case = wl.random_24_i8(np.random.default_rng(5), 64, 256, 128)
    c = dict(case, M=64, K=256, N=128)
    good = oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"])
    out = bench.cpu_baseline(c, perf, budget_s=0.01, gpu_out=good.copy())
    assert out["parity"]["bit_exact"] and out["parity"]["max_abs_diff"] == 0.0
    assert out["parity"]["elements"] == 64 * 128
    bad = good.copy()
    bad[3, 7] = np.nextafter(bad[3, 7], np.float32(np.inf))
    out = bench.cpu_baseline(c, perf, budget_s=0.01, gpu_out=bad)
    assert not out["parity"]["bit_exact"] and out["parity"]["max_abs_diff"] > 0
    assert "parity" not in bench.cpu_baseline(c, perf, budget_s=0.01)
