"""CPU oracle for precision flash attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP kernels are checked
against.  It shares no code with the GPU path and must never be imported by
the product package: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use it.

Parts
-----
numerics     BF16 round-to-nearest-even, FP32 rounding, hi/lo split.
attention64  Part A: plain attention forward and backward in float64.
flash_emu    Part B: tiled flash attention forward that rounds like the BF16
             kernel step by step, for the three modes (plain BF16 output, FP32
             output, repeated-maximum-aware safe softmax).
stats        Tolerance metrics, tie counts and the signed-error statistic.

Sources: "Why Low-Precision Transformer Training Fails: An Analysis on Flash
Attention" (arXiv 2510.04212) as summarised on paper-graph-ui, sections 3.4.2
to 3.4.5.
"""
