"""MI355X-native prefill MoE expert layer.

The layer runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
include/moe_prefill.h (libmoe_prefill.so).  ``quantized_expert_grouped_amd.abi`` is the thin
ctypes binding; it raises if the library has not been built.  ``synth`` holds the seeded
synthetic workloads.
"""
__all__ = ["abi", "synth"]
