"""Pins of the oracle's bf16 rounding against torch's CPU cast (a library routine)."""
import numpy as np
import torch

from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits


def _torch_bits(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_rne_matches_torch_sampled_bit_patterns():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties: low 16 bits 0x8000, 0x7FFF, 0x8001
    u[:300_000] = (u[:300_000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[300_000:400_000] = (u[300_000:400_000] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    u[400_000:500_000] = (u[400_000:500_000] & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    x = u.view(np.float32)
    ours = f32_to_bf16_bits(x)
    ref = _torch_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(bf16_bits_to_f32(ours[nan])))


def test_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.4e38, 1e-45, -1e-45,
                  1.0, 1.00390625, 1.005859375, 0.998046875], dtype=np.float32)
    ours = f32_to_bf16_bits(x)
    assert np.array_equal(ours, _torch_bits(x))
    # 0.998046875 = 1 - 2^-9 sits half-way between 0x3F7F and 0x3F80: ties go to even (1.0)
    assert ours[-1] == 0x3F80


def test_widen_is_exact():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f32(b)
    finite = np.isfinite(x)
    assert np.array_equal(f32_to_bf16_bits(x[finite]), b[finite])
