"""Pins of the W8A8-INT8 oracle.

Pins: closed forms for the per-token and per-channel scales (the largest
magnitude maps to +-127), ties to even, the zero row and column, the all-ones
product, an exhaustive check of the code map on a row that holds every
representable quotient and every midpoint, brute force over python integers on
tiny shapes, and the half-step error bound of round-to-nearest."""
import numpy as np
import pytest

from oracle import int8 as i8
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_per_token_closed_form():
    a = np.zeros((3, 256), dtype=np.float32)
    a[0, 7] = -2.0
    a[0, 9] = 1.0
    a[1, :] = 0.5
    q, s = i8.quant_act_per_token(_bits(a))
    assert s[0] == np.float32(2.0) / np.float32(127.0)
    assert q[0, 7] == -127 and q[0, 9] == 64           # 1 / (2/127) = 63.5 -> ties to even 64
    assert np.all(q[1] == 127) and s[1] == np.float32(0.5) / np.float32(127.0)
    assert s[2] == 0 and np.all(q[2] == 0)             # zero row (I2)


def test_per_channel_closed_form():
    w = np.zeros((128, 16), dtype=np.float32)
    w[3, 0] = 0.25
    w[5, 0] = -0.125                                  # exactly half of amax: 63.5 -> 64 (even)
    w[6, 0] = 0.25 * 3 / 127                          # 3 code steps, rounded through bf16
    q, s = i8.quant_weight_per_channel(_bits(w))
    assert s[0] == np.float32(0.25) / np.float32(127.0)
    assert q[3, 0] == 127 and q[5, 0] == -64
    assert q[6, 0] == 3
    assert s[1] == 0 and np.all(q[:, 1] == 0)


def test_ties_and_every_code_exhaustive():
    """A row with amax 127 has scale exactly 1: every integer quotient in
    [-127, 127] maps to itself and every midpoint to the even neighbour."""
    ints = np.arange(-127, 128, dtype=np.float32)
    mids = (np.arange(-127, 127, dtype=np.float32) + 0.5)
    row = np.concatenate([ints, mids])
    a = _bits(row[None, :])
    assert np.array_equal(bf16_bits_to_f32(a)[0], row)   # all exact in bf16
    q, s = i8.quant_act_per_token(a)
    assert s[0] == 1.0
    assert np.array_equal(q[0, :255], ints.astype(np.int8))
    lo = np.floor(mids)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(q[0, 255:], even.astype(np.int8))


def test_all_ones_product_is_exact():
    K, N = 512, 16
    qa, sa = i8.quant_act_per_token(_bits(np.ones((2, K))))
    qw, sw = i8.quant_weight_per_channel(_bits(np.ones((K, N))))
    assert np.all(qa == 127) and np.all(qw == 127)
    y = i8.gemm_ref(qa, sa, qw, sw)
    s1 = float(np.float32(1.0) / np.float32(127.0))
    assert np.all(y == 127 * 127 * K * s1 * s1)
    assert np.allclose(y, K, rtol=1e-6)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (3, 256, 32), (5, 384, 16)])
def test_bruteforce_tiny(M, K, N):
    a = synth.activations(M, K, seed=M + K)
    w = synth.weights(K, N, seed=K + N)
    qa, sa = i8.quant_act_per_token(a)
    qw, sw = i8.quant_weight_per_channel(w)
    assert np.allclose(i8.gemm_ref(qa, sa, qw, sw), i8.gemm_bruteforce(qa, sa, qw, sw), rtol=1e-13, atol=0)


def test_roundtrip_error_bound():
    """Round to nearest: |x - s q| <= s / 2 (plus the fp32 quotient's rounding)."""
    w = synth.weights(1024, 64, seed=9)
    qw, sw = i8.quant_weight_per_channel(w)
    x = bf16_bits_to_f32(w).astype(np.float64)
    err = np.abs(x - qw.astype(np.float64) * sw.astype(np.float64)[None, :])
    assert np.all(err <= sw.astype(np.float64)[None, :] * (0.5 + 1e-5))
    assert np.all(np.abs(qw.astype(int)) <= 127) and np.any(np.abs(qw) == 127)


def test_accumulator_bound():
    assert 127 * 127 * i8.MAX_K < 2 ** 31 <= 127 * 127 * (i8.MAX_K * 2)


def test_fp64_product_equals_the_integer_sum():
    """Extreme codes (+-127 everywhere, K at the bound's scale): the fp64
    product equals the exact integer sum computed with python integers."""
    rng = np.random.default_rng(5)
    K = 8192
    qa = rng.choice(np.array([-127, 127], dtype=np.int8), size=(2, K))
    qw = rng.choice(np.array([-127, -126, 125, 127], dtype=np.int8), size=(K, 3))
    y = i8.gemm_ref(qa, np.ones(2, np.float32), qw, np.ones(3, np.float32))
    for m in range(2):
        for n in range(3):
            assert y[m, n] == sum(int(a) * int(b) for a, b in zip(qa[m], qw[:, n]))
