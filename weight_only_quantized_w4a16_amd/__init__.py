"""MI355X (gfx950) quantized linear layer for LLM decode: W4A16 INT4-g128 and W8A8-FP8.

The compute lives in the HIP library libqgemm.so (C ABI declared in
include/qgemm.h); `ops` is a thin ctypes binding with the same entry-point
names.  Import `weight_only_quantized_w4a16_amd.ops` to load the library.
"""
__all__ = ["ops", "synth"]
