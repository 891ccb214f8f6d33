"""MI355X-native LongCat-Flash zero-computation-expert MoE layer.

The compute path is the HIP library `liblcmoe.so` (C ABI declared in
include/lcmoe.h); `mixture_experts_layer_biased_amd.lcmoe` is its thin ctypes
binding over torch device tensors. Submodules are imported on demand so that
`inputs` can be used without loading the library.
"""

__all__ = ["lcmoe", "inputs", "build"]
