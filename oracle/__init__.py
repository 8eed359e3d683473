"""CPU oracle for NVFP4 W4A4 linear layers -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP library is checked
against.  Only the test-suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path never
does, and the product path shares no code with it (no headers, tables,
helpers or constants).

What it computes, and where the pages say so
--------------------------------------------
Sources: the five web pages about arXiv 2609.04098, "Why Gated DeltaNet
Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid
27B LLM".

* Linear layers run with 4-bit weights and 4-bit activations ("W4A4") in
  NVIDIA's FP4 format, NVFP4 (bayesiansapien page, TL;DR; aipulsen page,
  second paragraph).
* NVFP4 uses 16-element block scaling, so one scale covers 16 elements and an
  outlier only affects its own block (bayesiansapien page, "The four-part
  mechanism study", first item; nefut page, first bullet).
* Per-module global scales exist, and fusing modules into one GEMM must keep
  them apart (bayesiansapien page, mechanism study, "Two practical repairs";
  nefut page, last paragraph; aimodeling page, "What engineers should
  actually take away").

The pages do not spell out the element code (E2M1), the scale code (E4M3),
the FP32 global scale, the amax/6 rule or round-to-nearest-even; the oracle
uses those standard NVFP4 choices and every reading taken is listed in the
module that takes it.

Modules
-------
``formats``   E2M1 / E4M3 code tables and round-to-nearest-even encoders.
``quantize``  vectorised numpy NVFP4 quantizer (FP32 arithmetic).
``scalar``    definitional scalar quantizer in exact rationals with an
              explicit IEEE binary32 rounding function (an independent
              second implementation used to pin ``quantize``).
``gemm``      fp64 dequantisation, W4A4 GEMM, the sum(|a*b|) error bound.
``epilogue``  fp64 SiLU*mul, sigmoid and Gated-DeltaNet decay epilogues.
``recurrence`` the gated delta-rule recurrence of a Gated DeltaNet layer
              (fp64), the second workload.
``mechanism`` the coarser-scaled reference formats (E4M3 scale per B
              elements; one per-tensor scale) and the error measures of the
              pages' mechanism study.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against brute force, closed forms, library routines or hand-worked examples;
none is "parity unpinned".
"""
