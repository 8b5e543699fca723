"""CPU oracle for the microscaling quantizers, dequantizers and block-scaled GEMMs.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path (the HIP library, its
Python binding) imports, calls or links anything in this package; only the
tests, the smoke check and the CPU-baseline leg of the benchmark do.  It shares
no code, tables or constants with the GPU sources.

Everything here is written to be checked by eye against the pages it follows:

* "Miles Blackwell RL Troca a Uniformidade BF16 por MXFP8 e NVFP4 Nativos"
  (remio.ai) -- MXFP8 = 32 E4M3 values under one E8M0 scale; NVFP4 = 16 E2M1
  values under one E4M3 scale plus a per-token FP32 scale; one fused op yields
  packed FP4, block scales and token scales; gate/up share one scale.
* "NVFP4 RL training" (The 4-bitter Lesson, socker-news.uzaya.net) --
  per-token activation scaling, dequantized backward y = x * DQ(Q(w)).
* "End-to-End MXFP8 Reinforcement Learning on Blackwell" (thelatestinai.com),
  Table 10 F6 -- E8M0 scales keep only an exponent.
* "Train models faster with JAX and MaxText using NVFP4 on NVIDIA Blackwell"
  (developer.nvidia.cn), section "NVFP4 pretraining recipe" -- 16x16 weight
  blocks shared by FPROP and DGRAD, 1x16 activation/gradient blocks, RNE for
  weights and activations, stochastic rounding for gradients, BF16 GEMM outputs.

Floating point: exact float64 wherever a step has an exact value; the NVFP4
scale chain is binary32 IEEE (round-to-nearest-even, subnormals kept, no fused
multiply-add), because there the floating-point result decides an integer code
and both sides must take that decision in the same precision.

Parity status: every function is pinned by a `-m "not gpu"` test against a
library routine, a closed form, a brute-force search or an invariant; none is
"parity unpinned".
"""

from . import formats, philox, mxfp8, nvfp4, layout, gemm, moe  # noqa: F401
