"""CPU oracle for the FP8 routed-expert MoE layer — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct fp64 reference for one GPU's
share of a routed-expert MoE layer under expert parallelism.  It exists only so
that tests, the smoke check and the benchmark's CPU-baseline leg can check and
time the HIP library against it.  The product path (the C-ABI library and its
Python binding) never imports, calls or links anything here, and nothing here
imports the product path.

Sources.  The method is the one described on two pages:

* "Deploying DeepSeek with PD Disaggregation and Large-Scale Expert Parallelism
  on 96 H100 GPUs" (LMSYS blog summary; called the *H100-EP page* below),
  sections "Large-scale expert parallelism / Expert parallelism with DeepEP"
  (token routing to experts, dispatch and combine) and "DeepGEMM integration"
  (FP8 grouped GEMMs for MoE, one per inference phase).
* "Deploying DeepSeek on GB200 NVL72 with PD and Large Scale EP (Part I): 2.7x
  Higher Decoding Throughput" (called the *GB200 page*), sections
  "How it is done" and "Method details" (FP8 GEMM library whose API quantises
  and packs input scales; DeepEP shuffling tokens to routed experts).

The pages fix the shape of the computation but not its arithmetic details
(block sizes, rounding, activation).  Every such detail is a stated reading,
listed in each function's docstring.

Modules:
  codec  - OCP E4M3FN encode/decode and bf16 rounding, bit-level, from the
           format definitions.
  moe    - block quantisation, layout (count / prefix-sum / stable rank),
           permute, grouped GEMM, SiLU-mul-requant, combine, chained layer.
  dense  - brute-force per-token dense MoE used only to pin `moe` on tiny
           inputs.

Pins: every function is checked by a CPU test under tests/ against
something other than itself -- exhaustive codec checks against torch's
casts, the fp32 block quantiser against torch's fp32 ops, Python-loop brute
force for the layout, permute and segment ranges, exact-integer and
power-of-two-scale GEMM cases, closed forms for the activation and the
combine, and a brute-force dense MoE for the whole layer (the test_oracle_*
modules list which pin covers which function).
"""

from . import codec, moe, dense  # noqa: F401
