"""Pins of the MSE-optimal-clipping quantizer of the oracle.

The clipping threshold alpha * max|x| is searched per group of 128 weights to
minimize the group's summed squared error ("Give Me BF16 or Give Me Death",
section 3.4, "W4A16-INT", paragraphs on MSE-optimal clipping).  Pins: the
one-point grid reduces to the abs-max quantizer, two groups whose optimum is
worked out by hand, an exact brute force over the grid in rational
arithmetic, and the invariants the definition implies (never worse than
abs-max, saturation beyond the threshold).
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import int4_g128 as q4
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_one_point_grid_is_abs_max():
    w = synth.weights(512, 48, seed=3)
    heavy = _bits(np.random.default_rng(4).standard_t(2, (512, 48)).astype(np.float32) * 0.02)
    for wb in (w, heavy):
        c1, s1 = q4.quantize_mse(wb, n_alpha=1)
        c0, s0 = q4.quantize(wb)
        assert np.array_equal(s1, s0)
        assert np.array_equal(c1, c0)


def test_outlier_group_worked_by_hand():
    # 127 weights of 1.0 and one of 8.0.  While the 1.0s take code 1 and the
    # 8.0 saturates at 7 the error is 127 (1 - s)^2 + (8 - 7 s)^2, minimal at
    # s = 366/352 = 1.0398; the nearest bf16 scales are 1.0390625 (error
    # 0.72168) and 1.046875 (0.73047).  bf16(8 * 91 / 700 = 1.04) = 1.0390625
    # (0x3F85), so alpha = 0.91 wins; abs-max (alpha = 1) gives s = 1.140625
    # and error 2.51172.
    w = np.ones((128, 16), dtype=np.float32)
    w[0, :] = 8.0
    codes, s = q4.quantize_mse(_bits(w))
    assert np.all(s == 0x3F85)
    assert np.all(codes[0] == 15) and np.all(codes[1:] == 9)
    err = q4.group_sq_error(_bits(w), codes, s)
    assert np.all(err == 127 * (1 - 1.0390625) ** 2 + (8 - 7 * 1.0390625) ** 2)
    c0, s0 = q4.quantize(_bits(w))
    assert np.all(s0 == 0x3F92)                      # bf16(8 / 7) = 1.140625
    assert np.all(q4.group_sq_error(_bits(w), c0, s0) == 127 * 0.140625 ** 2 + 0.015625 ** 2)


def test_equal_magnitudes_keep_abs_max():
    # every |x| = 1: q = +-7 and d = 1 - 7 s; the bf16 scale nearest 1/7 is
    # 0x3E12 (0.142578125, |d| = 2^-9), reached only at alpha = 1
    w = np.where(np.random.default_rng(0).random((256, 16)) < 0.5, -1.0, 1.0).astype(np.float32)
    codes, s = q4.quantize_mse(_bits(w))
    assert np.all(s == 0x3E12)
    assert set(np.unique(codes)) == {1, 15}
    assert np.all(q4.group_sq_error(_bits(w), codes, s) == 128 * 2.0 ** -18)


def _round_half_even(fr):
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    return fl


@pytest.mark.parametrize("n_alpha", [7, 100])
def test_exact_bruteforce_over_the_grid(n_alpha):
    """For each group and every grid point: the candidate scale, exact
    rational codes and exact squared error; the chosen scale is the exact
    minimizer (ties to the larger alpha) and the codes are its codes."""
    rng = np.random.default_rng(n_alpha)
    cols = [rng.standard_normal(128) * 0.02,
            rng.standard_t(2, 128) * 0.02,
            np.concatenate([rng.standard_normal(127) * 0.01, [0.3]]),
            rng.uniform(-1, 1, 128),
            np.concatenate([np.zeros(120), rng.standard_normal(8)]),
            np.zeros(128)]
    cols += [rng.standard_t(3, 128) for _ in range(10)]
    w = np.stack(cols, axis=1).astype(np.float32)
    wb = _bits(w)
    x = bf16_bits_to_f32(wb)
    codes, s_bits = q4.quantize_mse(wb, n_alpha=n_alpha)
    for n in range(w.shape[1]):
        xs = [Fraction(float(v)) for v in x[:, n]]
        amax = np.max(np.abs(x[:, n]))
        best = None
        for i in range(1, n_alpha + 1):
            q32 = np.float32(amax * np.float32(i)) / np.float32(7 * n_alpha)
            sb = int(f32_to_bf16_bits(np.array([q32]))[0])
            sv = Fraction(float(bf16_bits_to_f32(np.array([sb], dtype=np.uint16))[0]))
            if sv == 0:
                q = [0] * 128
            else:
                q = [min(7, max(-7, _round_half_even(v / sv))) for v in xs]
            err = sum((v - qq * sv) ** 2 for v, qq in zip(xs, q))
            if best is None or err <= best[0]:
                best = (err, sb, q)
        assert s_bits[0, n] == best[1], n
        assert np.array_equal(codes[:, n].astype(int) - 8, np.array(best[2])), n


def test_never_worse_than_abs_max_and_saturates_beyond_threshold():
    rng = np.random.default_rng(11)
    w = _bits(rng.standard_t(3, (1024, 64)).astype(np.float32) * 0.02)
    codes, s = q4.quantize_mse(w)
    c0, s0 = q4.quantize(w)
    e = q4.group_sq_error(w, codes, s)
    e0 = q4.group_sq_error(w, c0, s0)
    assert np.all(e <= e0)
    assert e.sum() < 0.9 * e0.sum()                 # heavy tails: clipping pays
    x = bf16_bits_to_f32(w).reshape(8, 128, 64)
    sv = bf16_bits_to_f32(s)[:, None, :]
    q = codes.astype(int).reshape(8, 128, 64) - 8
    beyond = np.abs(x) >= 7.5 * sv
    assert np.all(np.abs(q[beyond]) == 7)
    assert np.all(np.abs(q) <= 7)


def test_rejects_bad_grid():
    with pytest.raises(ValueError):
        q4.quantize_mse(np.zeros((128, 16), np.uint16), n_alpha=0)
