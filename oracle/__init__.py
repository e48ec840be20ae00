"""CPU oracle for the quantized MoE expert grouped GEMM (test infrastructure).

This package is test infrastructure only: it is imported by ``tests/``,
by ``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of
``bench.py``, and by nothing on the product path. It shares no code with
the HIP library or its Python binding and imports neither.

It is written for plain correctness, in numpy, from definitions:

* ``formats``  FP8 (OCP e4m3 / e5m2) and E8M0 decode tables built from the
  bit-field definitions, and a saturating round-to-nearest-even encoder
  that searches the table.
* ``quant``    amax per scaling unit, fp32 scales, codes, and the row-wise,
  column-wise (per-group, 128-aligned, zero-filled) and weight layouts for
  the tensorwise, delayed, 1x128 / 128x128 blockwise and MX (32-element,
  E8M0) recipes.
* ``delayed``  the delayed-scaling state (amax history, max algorithm).
* ``gemm``     dequantization and the grouped GEMM (forward, dgrad, wgrad)
  in float64, bf16 rounding of outputs, relative Frobenius error, SQNR.
* ``swiglu``   the SwiGLU activation between the two GEMMs in reproducible
  fp32 (correctly rounded operations only), rounded to bf16: the reference
  for the fused SwiGLU-then-quantize pass.

Every function states the passage of the source pages it follows. The
pages name the recipes and formats but print no formula beyond
"amax, then scale, then cast"; where they are silent the reading taken is
stated in the function's docstring. Functions without an independent
pin are marked "parity unpinned" (there are none at present).
"""
from . import formats, quant, delayed, gemm, swiglu  # noqa: F401
