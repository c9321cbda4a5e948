"""MI355X-native online-quantized W8A8 / W4A8 linear layer.

The compute path is a C-ABI HIP library (libcider.so, declared in
include/cider.h) built for gfx950; `w8a8_online_quantized_amd.cider` is its
thin Python binding (argument marshalling only). Importing the package does
not load the library; the binding loads it on first use and raises if it is
missing.
"""
__all__ = ["inputs", "cider"]
