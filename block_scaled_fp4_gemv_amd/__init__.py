"""Routed block-scaled (NVFP4 / MXFP4 / FP8) MoE layer forward for MI355X (gfx950)."""
