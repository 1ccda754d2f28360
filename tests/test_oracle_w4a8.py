"""Pins of the W4A8-FP8 oracle: closed forms (identity and all-ones weights),
brute force on tiny shapes, the special case of activations that are already
exact e4m3 values times a power of two (where the product reduces to the
W4A16 oracle's), and the grouped form against per-expert calls."""
import numpy as np
import pytest

from oracle import fp8_e4m3 as f8
from oracle import int4_g128 as q4
from oracle import w4a8
from oracle.bf16 import f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth


def _bits(v):
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_identity_weight_closed_form():
    # W = I (128 x 128): each column's group has one 1.0, s = bf16(1/7) = 0.142578125,
    # code 15, w_hat = 0.998046875 on the diagonal and 0 elsewhere
    K = 128
    codes, s = q4.quantize(_bits(np.eye(K)))
    a = synth.activations(3, K, seed=1)
    qa, sa = f8.quant_act_per_token(a)
    y = w4a8.gemm_ref(qa, sa, codes, s)
    expect = f8.e4m3_decode(qa) * 0.998046875 * sa.astype(np.float64)[:, None]
    assert np.array_equal(y, expect)


def test_all_ones_closed_form():
    K, N = 512, 16
    codes, s = q4.quantize(_bits(np.ones((K, N))))
    qa, sa = f8.quant_act_per_token(_bits(np.ones((2, K))))
    assert np.all(f8.e4m3_decode(qa) == 448.0)
    y = w4a8.gemm_ref(qa, sa, codes, s)
    assert np.all(y == 448.0 * 0.998046875 * K * float(sa[0]))
    assert np.allclose(y, 0.998046875 * K, rtol=1e-6)


def test_exact_e4m3_activations_reduce_to_w4a16():
    """Activations whose rows already hold e4m3 values with amax 448 quantize
    to themselves (s_a = 1): the product equals the W4A16 oracle's."""
    rng = np.random.default_rng(3)
    table = f8.e4m3_decode_table()
    finite = table[np.isfinite(table)]
    a = rng.choice(finite, size=(4, 256))
    a[:, 0] = 448.0
    qa, sa = f8.quant_act_per_token(_bits(a))
    assert np.all(sa == 1.0)
    w = synth.weights(256, 32, seed=4)
    codes, s = q4.quantize(w)
    assert np.array_equal(w4a8.gemm_ref(qa, sa, codes, s), q4.gemm_ref(_bits(a), codes, s))


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (3, 256, 16), (2, 384, 32)])
def test_bruteforce_tiny(M, K, N):
    a = synth.activations(M, K, seed=M + K)
    qa, sa = f8.quant_act_per_token(a)
    codes, s = q4.quantize(synth.weights(K, N, seed=K + N))
    assert np.allclose(w4a8.gemm_ref(qa, sa, codes, s), w4a8.gemm_bruteforce(qa, sa, codes, s),
                       rtol=1e-12, atol=1e-12)


def test_grouped_is_per_expert():
    K, N = 256, 16
    offsets = np.array([0, 2, 2, 7], dtype=np.int32)
    a = synth.activations(7, K, seed=5)
    qa, sa = f8.quant_act_per_token(a)
    ex = {e: q4.quantize(synth.weights(K, N, seed=50 + e)) for e in range(3)}
    y = w4a8.grouped_gemm_ref(qa, sa, offsets, ex)
    assert y[1].shape == (0, N)
    assert np.array_equal(y[2], w4a8.gemm_ref(qa[2:7], sa[2:7], *ex[2]))


def test_low_e4m3_bytes_are_the_nibble_values():
    """e4m3 bytes 0x00..0x0F decode to c * 2^-9 (subnormals 0..7, then the
    lowest binade 8..15): a stored 4-bit code read as an e4m3 byte is its own
    value scaled by 2^-9, so INT4 weights need no conversion table on the fp8
    MFMA."""
    t = f8.e4m3_decode_table()
    assert np.array_equal(t[:16], np.arange(16) * 2.0 ** -9)
    assert t[0x88] == -8 * 2.0 ** -9
