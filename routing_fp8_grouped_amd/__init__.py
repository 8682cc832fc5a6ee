"""MI355X (gfx950) forward pass of a DeepSeek-V3 MoE layer."""
