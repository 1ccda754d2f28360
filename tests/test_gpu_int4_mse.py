"""GPU parity of pack_int4_g128_mse (INT4 g128 with MSE-optimal clipping)
against the oracle: native words and scales bit-exact, at small shapes in
full and at full Llama-3 shapes on sampled columns; the abs-max special case
against pack_int4_g128; and a GEMM over MSE-packed weights within the GEMM
tolerance."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16, host_u32
from oracle import int4_g128 as q4
from oracle.bf16 import f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _heavy(K, N, seed, df=3):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits((rng.standard_t(df, (K, N)) * 0.02).astype(np.float32))


def _pack_mse(ops, w_bits, n_alpha):
    wt = ops.Int4G128Weight.from_bf16(dev_bf16(w_bits), mse_grid=n_alpha)
    torch.cuda.synchronize()
    return wt


@pytest.mark.parametrize("K,N,n_alpha,dist", [(128, 16, 100, "normal"), (512, 48, 100, "heavy"),
                                              (1280, 144, 100, "normal"), (1024, 272, 37, "heavy"),
                                              (256, 64, 1, "heavy"), (384, 32, 1000, "heavy")])
def test_pack_mse_bit_exact(ops, K, N, n_alpha, dist):
    announce(f"pack_int4_g128_mse K={K} N={N} n_alpha={n_alpha} {dist}")
    w = synth.weights(K, N, seed=K + 3 * N) if dist == "normal" else _heavy(K, N, seed=K + N)
    codes, s = q4.quantize_mse(w, n_alpha=n_alpha)
    packed_ref, scales_ref = q4.pack_native(codes, s)
    wt = _pack_mse(ops, w, n_alpha)
    assert np.array_equal(host_bits16(wt.scales), scales_ref)
    assert np.array_equal(host_u32(wt.packed), packed_ref)


def test_pack_mse_one_point_grid_equals_abs_max(ops):
    announce("pack_int4_g128_mse n_alpha=1 vs pack_int4_g128")
    w = _heavy(2048, 1024, seed=5)
    a = _pack_mse(ops, w, 1)
    b = ops.Int4G128Weight.from_bf16(dev_bf16(w))
    torch.cuda.synchronize()
    assert torch.equal(a.packed, b.packed) and torch.equal(a.scales, b.scales)


def test_pack_mse_special_groups(ops):
    """Zero groups, the hand-worked outlier group (alpha = 0.91, s = 0x3F85)
    and equal magnitudes (alpha = 1, s = 0x3E12)."""
    announce("pack_int4_g128_mse special groups")
    w = np.zeros((384, 32), dtype=np.float32)
    w[128:256, :] = 1.0
    w[128, :] = 8.0
    rng = np.random.default_rng(1)
    w[256:, :] = np.where(rng.random((128, 32)) < 0.5, -1.0, 1.0)
    wb = f32_to_bf16_bits(w)
    codes, s = q4.quantize_mse(wb)
    assert np.all(s[0] == 0) and np.all(s[1] == 0x3F85) and np.all(s[2] == 0x3E12)
    packed_ref, scales_ref = q4.pack_native(codes, s)
    wt = _pack_mse(ops, wb, 100)
    assert np.array_equal(host_bits16(wt.scales), scales_ref)
    assert np.array_equal(host_u32(wt.packed), packed_ref)


@pytest.mark.parametrize("name,K,N", [("qkv", 4096, 6144), ("down", 14336, 4096)])
def test_pack_mse_full_shape_sampled(ops, name, K, N):
    """Full Llama-3-8B shapes; the oracle quantizes sampled columns (each
    column's groups are independent), compared through the GPU dequant's
    code export and the native scale positions."""
    announce(f"pack_int4_g128_mse full {name} K={K} N={N}")
    w = _heavy(K, N, seed=13)
    wt = _pack_mse(ops, w, 100)
    _, codes_gpu = wt.dequant(with_codes=True)
    torch.cuda.synchronize()
    cols = np.unique(np.random.default_rng(7).integers(0, N, 24))
    codes, s = q4.quantize_mse(w[:, cols])
    assert np.array_equal(codes_gpu[:, cols].cpu().numpy(), codes)
    G = K // 128
    scales = host_bits16(wt.scales)
    idx = ((cols[None, :] // 16) * G + np.arange(G)[:, None]) * 16 + cols[None, :] % 16
    assert np.array_equal(scales[idx], s)


def test_gemm_over_mse_weights(ops):
    announce("qgemm_w4a16 over MSE-packed weights M=16 K=4096 N=512")
    w = _heavy(4096, 512, seed=21)
    a = synth.activations(16, 4096, seed=22)
    wt = _pack_mse(ops, w, 100)
    y = host_bits16(ops.W4A16Linear(wt)(dev_bf16(a)))
    codes, s = q4.quantize_mse(w)
    assert_close_rms(y, q4.gemm_ref(a, codes, s), what="gemm over MSE weights")
