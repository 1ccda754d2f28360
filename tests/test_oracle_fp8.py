"""Pins of the FP8 (OCP e4m3fn) oracle.

Pins: the 256-entry decode table against the format definition's landmarks and
against torch's float8_e4m3fn (a library routine); encoding against torch's
cast and against a brute-force nearest search; closed forms for the
per-token and per-channel scales; the all-ones product; brute force on tiny
shapes.
"""
import numpy as np
import pytest
import torch

from oracle import fp8_e4m3 as f8
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_decode_table_landmarks(golden):
    t = f8.e4m3_decode_table()
    assert t[0x7E] == golden("formats.txt")["e4m3_qmax"][0] == 448.0
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x38] == 1.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)


def test_decode_table_matches_torch():
    t = f8.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], ref[~nan])


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 500_000),
        rng.standard_normal(500_000) * 10.0,
        rng.standard_normal(200_000) * 1e-2,
        rng.standard_normal(100_000) * 1e-4,
    ]).astype(np.float32)
    # exact midpoints between neighbouring e4m3 values (ties) and the values themselves
    pos = f8.e4m3_decode_table()[:127]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32), -pos.astype(np.float32)])
    ours = f8.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_bruteforce_nearest_even():
    pos = f8.e4m3_decode_table()[:127]
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(0, 448, 3000), ((pos[1:] + pos[:-1]) / 2)]).astype(np.float32)
    codes = f8.e4m3_encode(x)
    for v, c in zip(x.astype(np.float64), codes):
        d = np.abs(pos - v)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want


def test_saturation_and_sign():
    x = np.array([448.0, 448.00003, 460.0, -448.00003, -1e-6, 0.0, -0.0], dtype=np.float32)
    assert list(f8.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


def test_per_token_closed_form():
    a = np.zeros((2, 128), dtype=np.float32)
    a[0, :3] = [1.0, -2.0, 0.5]
    q, s = f8.quant_act_per_token(_bits(a))
    assert s[0] == np.float32(2.0) / np.float32(448.0)
    # 1/s = 224 = 1.75*2^7 -> 0x76; -2/s = -448 -> 0xFE; 0.5/s = 112 -> 0x6E
    assert list(q[0, :3]) == [0x76, 0xFE, 0x6E]
    assert np.all(q[0, 3:] == 0)
    # an all-zero row: scale 0 and every code 0
    assert s[1] == 0 and np.all(q[1] == 0)


def test_per_channel_closed_form():
    w = np.zeros((128, 16), dtype=np.float32)
    w[:, 0] = 0.25
    w[7, 1] = -3.0
    q, s = f8.quant_weight_per_channel(_bits(w))
    assert s[0] == np.float32(0.25) / np.float32(448.0) and np.all(q[:, 0] == 0x7E)
    assert q[7, 1] == 0xFE and np.all(np.delete(q[:, 1], 7) == 0)
    assert np.all(s[2:] == 0) and np.all(q[:, 2:] == 0)


def test_all_ones_product_is_exact():
    M, K, N = 3, 4096, 16
    qa, sa = f8.quant_act_per_token(_bits(np.ones((M, K))))
    qw, sw = f8.quant_weight_per_channel(_bits(np.ones((K, N))))
    assert np.all(qa == 0x7E) and np.all(qw == 0x7E)
    assert np.all(sa == np.float32(1.0) / np.float32(448.0))
    y = f8.gemm_ref(qa, sa, qw, sw)
    # 448 * 448 * K * (1/448 rounded)^2 = K up to the fp32 rounding of 1/448
    assert np.allclose(y, K, rtol=1e-6)


def test_roundtrip_error_bound():
    """|x - s*dec(enc(x/s))| <= s * half-ulp of e4m3 at |x/s| (relative 2^-4 for normals)."""
    w = synth.weights(256, 64, seed=21)
    q, s = f8.quant_weight_per_channel(w)
    x = bf16_bits_to_f32(w).astype(np.float64)
    xr = f8.e4m3_decode(q) * s[None, :].astype(np.float64)
    v = np.abs(x / s[None, :])
    bound = np.where(v >= 2.0 ** -6, v * 2.0 ** -4, 2.0 ** -10) * s[None, :] * (1 + 1e-6)
    assert np.all(np.abs(x - xr) <= bound)


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (3, 256, 32), (16, 128, 16)])
def test_bruteforce_tiny(M, K, N):
    qa, sa = f8.quant_act_per_token(synth.activations(M, K, seed=31 + M))
    qw, sw = f8.quant_weight_per_channel(synth.weights(K, N, seed=41 + N))
    assert np.allclose(f8.gemm_ref(qa, sa, qw, sw), f8.gemm_bruteforce(qa, sa, qw, sw), rtol=1e-12, atol=1e-15)


def test_native_order_direct_formula():
    K, N = 256, 32
    qw, _ = f8.quant_weight_per_channel(synth.weights(K, N, seed=51))
    buf = f8.pack_native(qw)
    rng = np.random.default_rng(3)
    for k, n in zip(rng.integers(0, K, 1000), rng.integers(0, N, 1000)):
        nt, c = divmod(int(n), 16)
        kt, r = divmod(int(k), 128)
        half, r = divmod(r, 64)
        j, i = divmod(r, 16)
        assert buf[(nt * (K // 128) + kt) * 2048 + (16 * j + c) * 32 + 16 * half + i] == qw[k, n]
    assert np.array_equal(f8.unpack_native(buf, K, N), qw)
