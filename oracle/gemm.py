"""Oracle GEMMs (numpy, float64).  Test infrastructure only.

Both sparsity patterns reach exactly the product of A with the densified
pruned weight W_p (zeros at pruned positions), so the reference result is that
definition written out:

    C_ref[m, n] = sum_k A[m, k] * W_p[k, n]

* 2:4 pattern -- GPUSQ-ViT ("Boost Vision Transformer with GPU-Friendly
  Sparsity and Quantization"), abstract: weights pruned 2:4 and run in FP16,
  then quantised to integers for the integer 2:4 path.
* tile-wise pattern -- "Accelerating Sparse DNN Models without
  Hardware-Support via Tile-Wise Sparsity", run-time slide: the condensed
  tile GEMM reads A through offset_k and writes C through offset_n, so the
  columns of C outside a tile's kept set receive no contribution (zero).

Precision: fp16 inputs are converted exactly to float64 and multiplied with
numpy's BLAS; each fp16 x fp16 product is exact in float64 and the summation
error is below 2^-53 * K * sum|a||w|, negligible against fp16 output rounding.
int8 inputs give integer partial sums of magnitude <= K * 127 * 127 < 2^53, so
the float64 product is exact in any summation order.
"""

from __future__ import annotations

import numpy as np


def ref_gemm_f64(A, Wp):
    """C_ref = A . W_p in float64 (the masked dense product)."""
    A64 = np.asarray(A).astype(np.float64)
    W64 = np.asarray(Wp).astype(np.float64)
    if A64.ndim != 2 or W64.ndim != 2 or A64.shape[1] != W64.shape[0]:
        raise ValueError(f"shape mismatch {A64.shape} x {W64.shape}")
    return A64 @ W64


def ref_abs_gemm(A, Wp):
    """S = |A| . |W_p| in float64: the scale of the accumulated rounding error."""
    return np.abs(np.asarray(A).astype(np.float64)) @ np.abs(np.asarray(Wp).astype(np.float64))


def ref_gemm_f16(A, Wp):
    """fp16 path: (C_ref in float64, C_ref rounded once to fp16 with round-to-nearest-even).

    The kernels accumulate in fp32 and round the accumulator once to fp16; the
    float64 value is what parity is measured against.  numpy's float64 ->
    float16 conversion is correctly rounded (nearest, ties to even).
    """
    C64 = ref_gemm_f64(A, Wp)
    return C64, C64.astype(np.float16)


def ref_gemm_i8(A, Wp, scale=None):
    """int8 path (integer 2:4 GEMM of the GPUSQ-ViT abstract).

    acc[m, n] = sum_k A[m, k] * W_p[k, n] exactly (int32 range checked).
    With ``scale`` None the result is the int32 accumulator.  Otherwise
    C[m, n] = float32(acc[m, n]) * float32(scale[n]): one conversion with
    round-to-nearest-even, then one float32 multiply with round-to-nearest-even
    (no fused multiply-add, no bias, no clamp).
    """
    acc = ref_acc_i8(A, Wp)
    if scale is None:
        return acc
    return ref_i8_epilogue(acc, scale, None, "f32")


def ref_acc_i8(A, Wp):
    """Exact int32 accumulator of the int8 GEMM, sum_k A[m, k] * W_p[k, n]."""
    A = np.asarray(A)
    Wp = np.asarray(Wp)
    if A.dtype != np.int8 or Wp.dtype != np.int8:
        raise TypeError("int8 inputs expected")
    acc = ref_gemm_f64(A, Wp)
    acc_i = acc.astype(np.int64)
    if not np.array_equal(acc_i.astype(np.float64), acc):
        raise AssertionError("float64 integer sum was not exact")
    if acc_i.size and (acc_i.max() > 2**31 - 1 or acc_i.min() < -(2**31)):
        raise OverflowError("accumulator exceeds int32")
    return acc_i.astype(np.int32)


def ref_i8_epilogue(acc, scale, bias=None, out="f32"):
    """Epilogue of the integer path on the exact accumulator (the deployment
    outputs of the GPUSQ-ViT abstract's integer model: fp32, fp16 for the next
    fp16 layer, or requantised int8 for the next int8 layer).

        y[m, n] = float32(acc[m, n]) * scale[n]  (+ bias[n])

    each operation in float32 with round-to-nearest-even (conversion, product,
    sum; no fused multiply-add).  out: "f32" -> y; "f16" -> y rounded to the
    nearest fp16, ties to even, overflow to +-inf; "i8" -> y rounded to the
    nearest integer, ties to even, then saturated to [-128, 127]; "i32" -> the
    accumulator itself (no scale, no bias).
    """
    acc = np.asarray(acc)
    if acc.dtype != np.int32:
        raise TypeError("int32 accumulator expected")
    if out == "i32":
        if scale is not None or bias is not None:
            raise ValueError("the raw accumulator output takes no scale or bias")
        return acc.copy()
    if scale is None:
        raise ValueError("scale is required")
    y = acc.astype(np.float32) * np.asarray(scale, dtype=np.float32)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float32)[None, :]
    if out == "f32":
        return y
    if out == "f16":
        with np.errstate(over="ignore"):
            return y.astype(np.float16)
    if out == "i8":
        return np.clip(np.rint(y), -128, 127).astype(np.int8)
    raise ValueError(f"unknown output kind {out!r}")


def ref_gemm_i8_out(A, Wp, scale, bias=None, out="f16"):
    """int8 GEMM with the selectable epilogue: ref_i8_epilogue(ref_acc_i8(A, W_p), ...)."""
    return ref_i8_epilogue(ref_acc_i8(A, Wp), scale, bias, out)


def ref_tw_gemm_indexed(A, packed, N, G):
    """Tile-wise GEMM written with the slide's offset arrays, in float64.

    For tile t (output columns [t*G, t*G + G)) the condensed block V_t has
    N_t rows (kept columns, tile-local ids offset_n) and K_t columns (kept
    rows of W, global ids offset_k).  The tile contributes

        C[m, t*G + offset_n[j]] = sum_kk A[m, offset_k[kk]] * V_t[j, kk]

    and every other column of the tile's window stays zero ("Accelerating
    Sparse DNN Models without Hardware-Support via Tile-Wise Sparsity",
    run-time slide, indexed accesses of A, B and C).
    """
    A64 = np.asarray(A).astype(np.float64)
    M = A64.shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    vals = packed["vals"]
    ok, on = packed["offset_k"], packed["offset_n"]
    vp, kp, np_ = packed["v_ptr"], packed["k_ptr"], packed["n_ptr"]
    T = len(vp) - 1
    for t in range(T):
        kt = int(kp[t + 1] - kp[t])
        nt = int(np_[t + 1] - np_[t])
        if kt == 0 or nt == 0:
            continue
        ld = (int(vp[t + 1]) - int(vp[t])) // nt
        blk = vals[vp[t]:vp[t + 1]].reshape(nt, ld)[:, :kt].astype(np.float64)
        ks = ok[kp[t]:kp[t + 1]]
        ns = on[np_[t]:np_[t + 1]]
        C[:, t * G + ns] = A64[:, ks] @ blk.T
    return C


def ref_transpose(A):
    """K-major copy At[k, m] = A[m, k] (the tile-wise slides transpose A so the
    gathered rows are contiguous in memory)."""
    return np.ascontiguousarray(np.asarray(A).T)
