"""The oracle: a plain, slow, obviously correct CPU model of the sparse GEMM path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it.  The product path (the C-ABI
library and its Python binding) never imports, links or calls anything here,
and this package imports nothing from the product path: the two share no
code.  It depends on numpy alone.

What it computes (each function cites the passage it follows):

* ``gemm``      -- the masked dense product C = A . W_p on the densified pruned
  weights, in float64 (exact for int8 data), plus the int8 epilogues (fp32,
  fp16 or saturated int8 output of float32(acc) * scale (+ bias)) and the
  fp16 output rounding; the tile-wise indexed GEMM written with the slide's
  offset arrays.
* ``pack``      -- the 2:4 compressed format (kept values + 2-bit positions)
  and the tile-wise condensed format (tiles + offset_k / offset_n).
* ``bounds``    -- the error bounds that decide parity for floating point.

Pins: every function is checked in ``tests/test_oracle_*.py`` against
something other than itself (brute force with exact rationals on tiny
inputs, closed forms, invariants, special cases that reduce to a textbook
GEMM, and planted-mistake tests).  No function here is "parity unpinned".
"""

from .gemm import (  # noqa: F401
    ref_gemm_f64,
    ref_gemm_f16,
    ref_gemm_i8,
    ref_acc_i8,
    ref_i8_epilogue,
    ref_gemm_i8_out,
    ref_abs_gemm,
    ref_tw_gemm_indexed,
    ref_transpose,
)
from .pack import (  # noqa: F401
    ref_prune24_mask,
    ref_w24_positions,
    ref_w24_pack,
    ref_w24_unpack,
    ref_tw_structure,
    ref_tw_pack,
    ref_tw_unpack,
    TW_ROW_ALIGN_BYTES,
)
from .bounds import (  # noqa: F401
    loose_ok,
    loose_err,
    strict_bound_f16,
    strict_ok_f16,
)
