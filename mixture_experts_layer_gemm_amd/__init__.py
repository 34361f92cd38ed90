"""MI355X-native forward pass of one mixture-of-experts layer.

The compute lives in hand-written HIP kernels for gfx950 behind a C ABI
(``include/moe.h``); ``mixture_experts_layer_gemm_amd.moe`` is the thin Python binding
(argument marshalling only). Importing this package does not load the library;
importing ``.moe`` does, and fails loudly when it has not been built.
"""
__all__ = ["moe", "synth"]
