"""libs2attn: S2-Attn (LongLoRA shift short attention) forward and backward for MI355X."""
