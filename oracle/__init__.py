"""CPU oracle for one Beam-style MoE layer forward.  TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP path is checked
against.  Only the tests, the package smoke check and the bench's CPU
baseline may import it; the product path never does, and it shares no code
with the HIP kernels or their binding.

Sources (the three pages the method is described on):
  [TS] "TokenSpeed x Reflection Beam" (lightseek.org blog): sections
       "Architecture", "NVFP4 and FP8 checkpoints", "Fused FP32 routing",
       "MNNVL all-reduce and SandwichNorm fusion", "TensorRT-LLM NVFP4 MoE".
  [GD] "Beam-1.0-501B-A23B on Gaudi 2" (Gaudi cookbook): "What was built",
       "Correctness", "EP vs TP quality".
  [VL] agentlenshq.com (Korean) summary of vLLM's "Reflection Beam 1.0"
       day-0 post: section "MoE and residual stream: FP32 router, sandwich
       norm, depth-scaled residual" and the list of seven kernel changes.

Every function in oracle.moe cites the passage it follows.  Pins (checks of
the oracle against something other than itself) live in tests/test_oracle_*.
"""

from .moe import *  # noqa: F401,F403
