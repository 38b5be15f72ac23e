"""Block-scaled FP8 (W8A16) routed MoE expert FFN for AMD Instinct MI355X (gfx950).

The compute path lives in the HIP library ``libmoe_w8a16.so`` (C ABI in
``include/moe_w8a16.h``); ``block_scaled_fp8_amd.binding`` is its thin Python
binding.  ``block_scaled_fp8_amd.synth`` draws seeded synthetic inputs.
"""

__all__ = ["binding", "synth", "build"]
