"""CPU oracle for the block-scaled quantize + GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the benchmark's CPU-baseline leg use it.

It is a plain, slow, step-by-step NumPy implementation of what the method
computes, written from the source pages:

* "NVFP4 pretraining post" -- the NVIDIA blog text on NVFP4 pretraining with
  TransformerEngine/MaxText, section "NVFP4 pretraining recipe" (its five
  ingredients: 16-element micro-blocks, E4M3 block scales under a per-tensor
  FP32 scale, a Random Hadamard Transform on WGRAD inputs only, 16x16 2D
  weight scaling, stochastic rounding on gradients) and the data-flow
  paragraph after Figure 1 (FPROP / DGRAD / WGRAD consume NVFP4 inputs and
  emit BF16 outputs).
* "HN page opcode84" -- quotes the Triton-on-Blackwell blog on MXFP8 and
  MXFP4 GEMMs and links the OCP Microscaling Formats spec, which defines the
  E2M1 / E4M3 element types and the E8M0 power-of-two block scale.
* Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
  SC'11 -- the Philox4x32-10 counter-based generator used for stochastic
  rounding.

All FP32 steps are separate IEEE round-to-nearest-even NumPy float32 ops (no
fused multiply-add), subnormals kept, signed zeros preserved.  The GEMM is the
plain FP64 definition over dequantized operands.

Parity pins: every function here is pinned by tests under tests/ marked
"not gpu" (closed forms, exhaustive tables, library cross-checks, brute
force).  No function is "parity unpinned".
"""

from . import formats, philox, rht, quantize, gemm  # noqa: F401
