"""bfloat16 rounding for the oracle (test infrastructure only).

The pages keep weights, activations and the INT4 group scales in bf16
("When quantization pays -- and when it does not", section "Counting c from the
kernel, not from intuition": the conversion targets nv_bfloat162 pairs).  The
rounding used everywhere in the oracle is IEEE round-to-nearest-even from
fp32, written with integer bit operations.

Pinned by tests/test_oracle_bf16.py against torch's CPU bf16 cast (a library
routine) over sampled and special fp32 bit patterns.
"""
import numpy as np


def f32_to_bf16_bits(x):
    """Round fp32 values to bf16, nearest-even; return the uint16 bit patterns.

    NaN stays NaN (quieted); overflow rounds to +-inf as IEEE prescribes.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(x)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    out = np.where(nan, quiet, rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bf16 bit patterns (uint16) to fp32 values (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x):
    """fp32 -> nearest-even bf16 -> fp32 (the value a bf16 store keeps)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
