"""CPU oracle of the Kimi K3 Stable LatentMoE FFN forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP path; both read the canonical
bytes produced by the seeded generator module `synth`.

The oracle is written from the pages' description of the layer (the latent
mixture-of-experts block card of Kimi K3, "All 23 steps" and its code excerpt
of `KimiSparseMoeBlock.forward` / `moe_infer`; the Stable LatentMoE chapter of
the toy reproduction; the Chinese walkthrough of report section 2.3 and
Appendix B; the NVFP4 port notes) in float64, on exactly dequantised weights.
"""
from .moe_oracle import *  # noqa: F401,F403
from .qb import *  # noqa: F401,F403,E402
