"""Few-row block-quantized GEMV for MI355X (gfx950): q8 (Q8_0 / Q4_0) and f16 lanes.

The compute runs in hand-written HIP kernels behind a C ABI (include/qgemv.h,
built as block_quantized_few_amd/libqgemv.so).  This package holds the thin
ctypes binding (`qgemv`) and the seeded input generator (`synth`).  Importing
the package loads nothing native; the binding loads the library on first use
and raises if it is missing.
"""
