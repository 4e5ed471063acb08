"""Parity tolerances for the floating-point paths.  Test infrastructure only.

Loose bound (the acceptance bar for fp16 inputs with fp32 accumulation):

    max |C - C_ref| <= 1e-2 * max |C_ref|,   evaluated in float64, NaN fails.

Strict per-element bound, derived from the arithmetic the kernels perform
(fp16 x fp16 products are exact in fp32; n products are summed in fp32 in
some order; the fp32 sum is rounded once to fp16):

    |C - C_ref| <= u16 * |C_ref| + eta16 + (1 + u16) * 2 * n * u32 * S

with u16 = 2^-11 (fp16 unit roundoff), eta16 = 2^-25 (half the fp16
subnormal spacing), u32 = 2^-24 and S = |A| . |W_p|.  The factor 2 * n * u32
bounds the error of n fp32 additions in any order even if the matrix unit
does not round to nearest at every step; n is the number of products one
output sums (K for a dense GEMM, K/2 kept slots for 2:4, K_t of the output's
tile for tile-wise).  Since S is n times the average |a w| of the sum, the
bound catches a dropped or duplicated term larger than 2 n^2 u32 average
terms plus the output rounding: 0.018 of an average term at n = 384 (which
the loose bound can hide), half of one at n = 2048.  Smaller single terms can
sit inside a valid summation error, which is why exact-integer cases
(bit-exact whatever the summation order) pin the index paths.
"""

from __future__ import annotations

import numpy as np

U16 = 2.0 ** -11
ETA16 = 2.0 ** -25
U32 = 2.0 ** -24


def loose_err(C, C_ref):
    """max|C - C_ref| / max|C_ref| in float64 (inf if C has a NaN)."""
    C = np.asarray(C, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    if not np.isfinite(C).all():
        return float("inf")
    denom = float(np.abs(C_ref).max()) if C_ref.size else 0.0
    num = float(np.abs(C - C_ref).max()) if C_ref.size else 0.0
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / denom


def loose_ok(C, C_ref, tol=1e-2):
    return loose_err(C, C_ref) <= tol


def strict_bound_f16(C_ref, S, n):
    C_ref = np.asarray(C_ref, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    return U16 * np.abs(C_ref) + ETA16 + (1.0 + U16) * 2.0 * n * U32 * S


def strict_ok_f16(C, C_ref, S, n):
    """True iff every element of C meets the strict bound (and C is finite)."""
    C = np.asarray(C, dtype=np.float64)
    if not np.isfinite(C).all():
        return False
    return bool((np.abs(C - np.asarray(C_ref, dtype=np.float64)) <= strict_bound_f16(C_ref, S, n)).all())
