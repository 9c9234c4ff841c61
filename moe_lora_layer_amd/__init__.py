"""Fused MoE multi-LoRA layer for AMD MI355X (gfx950).

The compute path is the C-ABI library libmoelora.so (hand-written HIP kernels);
``moe_lora_layer_amd.ops`` is its thin Python binding.  Importing the package
does not load the library; the binding loads it on first use and raises if it
is missing.
"""
__all__ = ["ops", "synth"]
