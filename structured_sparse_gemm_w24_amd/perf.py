"""Work and traffic models plus report arithmetic (host-only, no GPU).

Algorithmic work is what the method itself must compute or move, not the
dense work it avoids:

* 2:4 GEMM: nonzero ops M*N*K (= half of the dense 2*M*N*K); bytes
  M*K*sA (activations) + N*K/2*sW (kept values) + N*K/8 (2-bit positions)
  + 4*N (per-channel scale, int8 only) + M*N*sC (output).
* tile-wise GEMM: nonzero flops 2*M*sum_t(K_t*N_t); bytes M*|union of kept
  rows|*2 (gathered activations, each row read once from HBM) + the condensed
  tiles as stored + the index arrays + M*N*2 (every output column is written,
  pruned columns as zeros).
* dense GEMM: 2*M*N*K; bytes M*K*sA + K*N*sW + M*N*sC (+4*N).
* transpose: 2*M*K*2 bytes.

Peaks are MI355X's published dense figures (HBM3E 8 TB/s; MFMA fp16
2.5 PFLOP/s, int8 5.0 POP/s).  Sparse-MFMA work is priced in nonzero
operations against the dense peak, so a fraction of 1.0 means the sparse
matrix core ran at its full 2x dense-equivalent rate.
"""

from __future__ import annotations

PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_I8_TOPS = 5000.0


def speedup(t_base, t_x):
    return t_base / t_x


def share(t_part, t_total):
    return t_part / t_total


def w24_ops(M, N, K):
    """(nonzero ops, dense-equivalent ops)."""
    return M * N * K, 2 * M * N * K


def w24_bytes(M, N, K, s_a, s_w, s_c, scale=False):
    return M * K * s_a + N * (K // 2) * s_w + N * K // 8 + (4 * N if scale else 0) + M * N * s_c


def dense_ops(M, N, K):
    return 2 * M * N * K


def dense_bytes(M, N, K, s_a, s_w, s_c, scale=False):
    return M * K * s_a + K * N * s_w + M * N * s_c + (4 * N if scale else 0)


def tw_ops(M, sum_kt_nt):
    return 2 * M * sum_kt_nt


def tw_bytes(M, N, union_rows, vals_elems, sum_kt, sum_nt, T):
    return M * union_rows * 2 + 2 * vals_elems + 4 * (sum_kt + sum_nt + 3 * (T + 1) + T) + M * N * 2


def transpose_bytes(M, K):
    return 2 * M * K * 2


def roofline(achieved, peak, unit, bound, traffic=None):
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic}


def bound_report(ops, bytes_, t_ms, peak_ops):
    """Ideal times at the MFMA peak (peak_ops, ops/s) and at the HBM peak, the
    bound that binds (the larger), and the roofline fraction ideal / measured."""
    t_mfma = ops / peak_ops
    t_hbm = bytes_ / (PEAK_HBM_GBS * 1e9)
    t = t_ms * 1e-3
    return {"t_ideal_mfma_us": t_mfma * 1e6, "t_ideal_hbm_us": t_hbm * 1e6,
            "bound": "mfma" if t_mfma >= t_hbm else "hbm", "roofline_frac": max(t_mfma, t_hbm) / t}
