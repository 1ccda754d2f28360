"""Pins of the INT4 g128 oracle against what the pages and arithmetic fix.

Pins: closed forms for the scale and codes, the identity and all-ones products,
4.125 stored bits per weight, the magic-number unpack constants the first page
prints, an exhaustive dequantization check against torch's bf16 cast, brute
force on tiny shapes, and invariance under permuting whole groups.
"""
import numpy as np
import pytest
import torch

from oracle import int4_g128 as q4
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_scale_of_unit_group_closed_form():
    # amax = 1: s = bf16(1/7) = 0x3E12 = 0.142578125
    w = np.zeros((128, 16), dtype=np.float32)
    w[5, 3] = 1.0
    codes, s = q4.quantize(_bits(w))
    assert s[0, 3] == 0x3E12
    assert bf16_bits_to_f32(s)[0, 3] == np.float32(0.142578125)
    # 1 / 0.142578125 = 7.0137 -> 7 -> stored code 15
    assert codes[5, 3] == 15
    wf = q4.dequant_f32(codes, s)
    assert wf[5, 3] == np.float32(0.998046875)
    # 0.998046875 = 1 - 2^-9 is a tie between 0x3F7F and 0x3F80: ties go to even -> 1.0
    assert q4.dequant_bf16_bits(codes, s)[5, 3] == 0x3F80


def test_zero_group_and_single_nonzero():
    w = np.zeros((256, 16), dtype=np.float32)
    w[130, 0] = 0.5
    w[131, 1] = -0.5
    codes, s = q4.quantize(_bits(w))
    # group 0 of every column and group 1 of columns >= 2 are zero: scale 0, code 8
    assert np.all(s[0] == 0) and np.all(codes[:128] == 8)
    assert np.all(s[1, 2:] == 0)
    assert codes[130, 0] == 15 and codes[131, 1] == 1       # +7 + 8 and -7 + 8
    other = np.ones_like(codes, dtype=bool)
    other[130, 0] = other[131, 1] = False
    assert np.all(codes[other] == 8)
    assert np.all(q4.dequant_f32(codes, s)[other] == 0)


def test_codes_stay_in_abs_max_range():
    w = synth.weights(512, 64, seed=11)
    codes, s = q4.quantize(w)
    assert codes.min() >= 1 and codes.max() <= 15         # -8 unused under abs-max
    # every nonzero group reaches +-7 at its abs-max element
    q = codes.astype(int).reshape(4, 128, 64) - 8
    assert np.all(np.abs(q).max(axis=1) == 7)


def test_rounding_ties_to_even():
    # group amax 7*2^-3 -> s = 0.125 exactly; w = 0.0625 -> w/s = 0.5 -> 0; w = 0.1875 -> 1.5 -> 2
    w = np.zeros((128, 16), dtype=np.float32)
    w[0, 0] = 0.875
    w[1, 0] = 0.0625
    w[2, 0] = 0.1875
    w[3, 0] = -0.0625
    w[4, 0] = -0.3125   # -2.5 -> -2
    codes, s = q4.quantize(_bits(w))
    assert bf16_bits_to_f32(s)[0, 0] == np.float32(0.125)
    assert list(codes[:5, 0].astype(int) - 8) == [7, 0, 2, 0, -2]


def test_density_4_125_bits(golden):
    g = golden("formats.txt")
    bits = g["bits_per_weight_g128"][0]
    for _, K, N in set(synth.LLAMA3_8B_LAYER) | set(synth.LLAMA3_70B_LAYER) | {synth.LLAMA3_8B_HEAD[:3], synth.LLAMA3_70B_HEAD[:3]}:
        assert q4.stored_bytes(K, N) * 8 == bits * K * N
    assert g["scale_overhead_bits"][0] == 16 / 128
    # the page's rounded 0.5156 bytes per weight
    assert abs(bits / 8 - g["bytes_per_weight_g128"][0]) < 5e-5
    # the 8B stack with the LM head
    total = sum(q4.stored_bytes(K, N) for _, K, N in synth.stack_shapes("8b"))
    assert total == 3_869_589_504


def test_magic_number_unpack_constants(golden):
    g = golden("formats.txt")
    mask, magic, sub = g["nibble_mask"][0], g["bf16_magic_pair"][0], g["bf16_offset_pair"][0]
    for n in range(16):
        word = (((n << 16) | n) & mask) | magic
        lo = np.array([word & 0xFFFF], dtype=np.uint16)
        hi = np.array([word >> 16], dtype=np.uint16)
        assert bf16_bits_to_f32(lo)[0] == 128 + n
        assert bf16_bits_to_f32(hi)[0] == 128 + n
        off = bf16_bits_to_f32(np.array([sub & 0xFFFF], dtype=np.uint16))[0]
        assert off == 136.0
        # the subtraction is exact in bf16: (128+n) - 136 = n - 8
        diff = torch.tensor([128.0 + n], dtype=torch.bfloat16) - torch.tensor([136.0], dtype=torch.bfloat16)
        assert float(diff) == n - 8


def test_dequant_exhaustive_codes_times_all_bf16_scales():
    s_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = bf16_bits_to_f32(s_bits)
    s_bits = s_bits[np.isfinite(s)]
    G = s_bits.size // 16                 # whole groups of 16 columns
    s_bits = s_bits[:G * 16]
    K = 128 * 16
    # one column block per scale, every code 0..15 present in each column
    codes = np.tile(np.repeat(np.arange(16, dtype=np.uint8), 8)[:, None], (16, 1))[:K]
    codes = np.tile(codes, (1, 16))
    for chunk in range(0, G, 512):
        sb = s_bits[chunk * 16:(chunk + 512) * 16]
        ncol = sb.size
        c = np.tile(codes[:128, :1], (1, ncol))
        scales = sb.reshape(1, ncol)
        with np.errstate(over="ignore"):
            wf = q4.dequant_f32(c, scales)
        exact = (c.astype(np.float64) - 8) * bf16_bits_to_f32(scales).astype(np.float64)
        fits = np.abs(exact) <= np.finfo(np.float32).max
        # the fp32 product is exact wherever it fits (at most 3 + 8 significant bits) ...
        assert np.array_equal(wf[fits].astype(np.float64), exact[fits])
        # ... and overflows to a signed infinity where it does not
        assert np.array_equal(wf[~fits], np.sign(exact[~fits]) * np.inf)
        ref = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(q4.dequant_bf16_bits(c, scales), ref)


def test_identity_weight_closed_form():
    K = N = 256
    w = np.eye(K, dtype=np.float32)
    codes, s = q4.quantize(_bits(w))
    a = synth.activations(3, K, seed=5)
    y = q4.gemm_ref(a, codes, s)
    assert np.array_equal(y, 0.998046875 * bf16_bits_to_f32(a).astype(np.float64))
    # with the bf16-rounded operand the identity is reproduced exactly
    assert np.array_equal(q4.gemm_ref_bf16_operand(a, codes, s), bf16_bits_to_f32(a).astype(np.float64))


def test_all_ones_closed_form():
    K, N, M = 4096, 16, 2
    codes, s = q4.quantize(_bits(np.ones((K, N))))
    a = _bits(np.ones((M, K)))
    y = q4.gemm_ref(a, codes, s)
    assert np.all(y == 4088.0)                       # 4096 * 0.998046875
    assert np.all(f32_to_bf16_bits(y.astype(np.float32)) == _bits([4096.0])[0])   # a tie -> even


@pytest.mark.parametrize("M", [1, 2, 3, 4, 16])
@pytest.mark.parametrize("K,N", [(128, 16), (256, 64)])
def test_bruteforce_tiny(M, K, N):
    a = synth.activations(M, K, seed=100 + M)
    codes, s = q4.quantize(synth.weights(K, N, seed=200 + K + N))
    y = q4.gemm_ref(a, codes, s)
    yb = q4.gemm_bruteforce(a, codes, s)
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_group_permutation_invariance():
    M, K, N = 4, 512, 32
    a = synth.activations(M, K, seed=3)
    w = synth.weights(K, N, seed=4)
    perm = np.array([2, 0, 3, 1])
    rows = np.concatenate([np.arange(128 * p, 128 * p + 128) for p in perm])
    c1, s1 = q4.quantize(w)
    c2, s2 = q4.quantize(w[rows])
    assert np.array_equal(s2, s1[perm])
    y1 = q4.gemm_ref(a, c1, s1)
    y2 = q4.gemm_ref(a[:, rows], c2, s2)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-13)
    # moving a single row across a group boundary does change the result
    swap = np.arange(K)
    swap[[0, 128]] = swap[[128, 0]]
    c3, s3 = q4.quantize(w[swap])
    assert not np.allclose(q4.gemm_ref(a[:, swap], c3, s3), y1, rtol=1e-6, atol=1e-9)


def _native_position(k, n, K):
    """Second statement of the native order: where (k, n) lives, computed directly."""
    G = K // 128
    nt, c = divmod(n, 16)
    g, r = divmod(k, 128)
    t, r = divmod(r, 32)
    j, i = divmod(r, 8)
    lane = 16 * j + c
    slot = i // 2 if i % 2 == 0 else 4 + i // 2
    return (nt * G + g) * 256 + lane * 4 + t, 4 * slot


def test_native_packing_matches_direct_position_formula():
    K, N = 384, 48
    codes, s = q4.quantize(synth.weights(K, N, seed=9))
    packed, sn = q4.pack_native(codes, s)
    assert packed.size * 4 + sn.size * 2 == q4.stored_bytes(K, N)
    rng = np.random.default_rng(0)
    for k, n in zip(rng.integers(0, K, 2000), rng.integers(0, N, 2000)):
        w, sh = _native_position(int(k), int(n), K)
        assert (int(packed[w]) >> sh) & 0xF == codes[k, n]
        assert sn[(n // 16 * (K // 128) + k // 128) * 16 + n % 16] == s[k // 128, n]
    c2, s2 = q4.unpack_native(packed, sn, K, N)
    assert np.array_equal(c2, codes) and np.array_equal(s2, s)


def test_native_word_yields_consecutive_bf16_pairs():
    """(word >> 4j) & 0x000F000F holds rows 2j (low half) and 2j+1 (high half)."""
    K, N = 128, 16
    codes, s = q4.quantize(synth.weights(K, N, seed=12))
    packed, _ = q4.pack_native(codes, s)
    for lane in range(64):
        for t in range(4):
            word = int(packed[lane * 4 + t])
            kb = 32 * t + 8 * (lane // 16)
            n = lane % 16
            for j in range(4):
                pair = (word >> (4 * j)) & 0x000F000F
                assert pair & 0xF == codes[kb + 2 * j, n]
                assert pair >> 16 == codes[kb + 2 * j + 1, n]


def test_canonical_packing():
    K, N = 256, 16
    codes, _ = q4.quantize(synth.weights(K, N, seed=13))
    words = q4.pack_canonical(codes)
    for k in range(K):
        assert np.array_equal((words[k // 8] >> np.uint32(4 * (k % 8))) & np.uint32(0xF), codes[k])
