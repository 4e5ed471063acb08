"""Structured-sparse weight GEMM for AMD Instinct MI355X (gfx950).

C = A x W for pruned linear layers, with W sparse in one of two patterns:

* 2:4 along K (at most two nonzeros in every four consecutive K entries of
  an output column), fp16 with fp32 accumulation and int8 with int32
  accumulation plus a per-output-channel fp32 scale;
* tile-wise: every G-column tile keeps its own K-rows and N-columns and runs
  as a condensed dense tile addressed through offset_k / offset_n.

The heavy lifting lives in the C-ABI library ``libssg.so`` (host packers and
hand-written gfx950 HIP kernels).  This package is a thin ctypes binding with
the same function names; it marshals numpy arrays (pack stage) and torch
device tensors (GEMMs) and raises ``SsgError`` on a nonzero status.  There is
no fallback: if the library is missing every call raises.
"""

from ._lib import (  # noqa: F401
    SsgError,
    lib_path,
    load,
    w24_pack_f16,
    w24_pack_i8,
    w24_unpack_f16,
    w24_unpack_i8,
    tw_pack_query,
    tw_pack_f16,
    tw_unpack_f16,
    tw_pack_i8,
    tw_unpack_i8,
    dense_gemm_f16,
    dense_gemm_i8,
    dense_gemm_i8_out,
    w24_gemm_f16,
    w24_gemm_i8,
    w24_gemm_i8_out,
    dense_gemm_f16_splitk,
    w24_gemm_f16_splitk,
    dense_gemm_i8_splitk,
    w24_gemm_i8_splitk,
    w24_gemm_f16_splitk_static,
    SSG_STATIC_SCRATCH_BYTES,
    splitk_suggest,
    tile_choice,
    splitk_workspace_bytes,
    SSG_KIND_DENSE_F16,
    SSG_KIND_W24_F16,
    SSG_KIND_DENSE_I8,
    SSG_KIND_W24_I8,
    SSG_OUT_I32,
    SSG_OUT_F32,
    SSG_OUT_F16,
    SSG_OUT_I8,
    tw_gemm_f16,
    tw_gemm_f16_ex,
    tw_gemm_i8,
    tw_gemm_f16_streams,
    SSG_TW_OUT_T,
    SSG_TW_A_ROWMAJOR,
    SSG_TW_NARROW,
    ssg_transpose_f16,
    ssg_device_arch,
    TwPacked,
)
from . import perf  # noqa: F401
