"""MI355X-native quantized attention forward (SageAttention family).

The compute path is the C-ABI library ``libsage.so`` (hand-written HIP kernels for
gfx950); ``bit_quantized_attention_03_amd.sage`` binds it.  Importing this package does not
load the library; ``sage`` does, and raises if it is missing.
"""
__all__ = ["inputs", "sage"]
