"""GPU parity of the W8A8-FP8 path against the CPU oracle.

Activation codes and scales, weight codes (native order) and scales:
bit-exact.  GEMM: max |err| <= 2e-2 x RMS of the fp64 oracle output.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16, host_u8
from oracle import fp8_e4m3 as f8
from oracle.bf16 import f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _act_quant(ops, a_bits):
    qa, sa = ops.quantize_activations(dev_bf16(a_bits))
    torch.cuda.synchronize()
    return host_u8(qa), sa.cpu().numpy()


# K spans every launch form: one wave per row (K <= 2048, 4096, 8192), one
# workgroup per row (14336, 28672) and the two-pass kernel for longer rows
@pytest.mark.parametrize("M,K", [(1, 128), (4, 4096), (16, 14336), (37, 1000), (256, 4096), (3, 8192),
                                 (5, 28672), (2, 40960)])
def test_act_quant_bit_exact(ops, M, K):
    announce(f"quant_act_per_token M={M} K={K}")
    a = synth.activations(M, K, seed=M + K)
    q, s = _act_quant(ops, a)
    q_ref, s_ref = f8.quant_act_per_token(a)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_act_quant_ties_subnormals_and_zero_rows(ops):
    """Rows with amax 448 (scale exactly 1): every e4m3 value, every midpoint
    between neighbours (ties to even), the subnormal range, signs, and zero rows."""
    announce("quant_act_per_token ties / subnormals / zero rows")
    pos = f8.e4m3_decode_table()[:127]
    mids = (pos[1:] + pos[:-1]) / 2
    vals = np.concatenate([pos, mids, -pos, -mids, [0.0, -0.0, 1e-6, -1e-6, 2.0 ** -11, 3 * 2.0 ** -11]])
    K = 512
    rows = []
    for start in range(0, vals.size, K - 1):
        r = np.zeros(K)
        chunk = vals[start:start + K - 1]
        r[:chunk.size] = chunk
        r[-1] = 448.0
        rows.append(r)
    rows.append(np.zeros(K))                       # an all-zero row
    small = np.zeros(K)
    small[:5] = [3e-3, -7e-4, 1e-5, 2.5e-3, -1e-6]  # a row of tiny values (scale ~ 7e-6)
    rows.append(small)
    a = f32_to_bf16_bits(np.array(rows, dtype=np.float32))
    q, s = _act_quant(ops, a)
    q_ref, s_ref = f8.quant_act_per_token(a)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("K,N", [(128, 16), (384, 48), (4096, 4096), (14336, 4096)])
def test_weight_quant_bit_exact(ops, K, N):
    announce(f"quant_weight_fp8_per_channel K={K} N={N}")
    w = synth.weights(K, N, seed=K * 3 + N)
    fw = ops.Fp8Weight.from_bf16(dev_bf16(w))
    torch.cuda.synchronize()
    qw_ref, sw_ref = f8.quant_weight_per_channel(w)
    assert np.array_equal(fw.scales.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    got = host_u8(fw.codes)
    if K * N <= 4096 * 4096:
        assert np.array_equal(got, f8.pack_native(qw_ref))
    else:
        assert np.array_equal(f8.unpack_native(got, K, N)[:, :64], qw_ref[:, :64])
        rng = np.random.default_rng(0)
        k = rng.integers(0, K, 200000)
        n = rng.integers(0, N, 200000)
        r = k % 128
        idx = ((n // 16) * (K // 128) + k // 128) * 2048 + (16 * ((r % 64) // 16) + n % 16) * 32 \
            + 16 * (r // 64) + r % 16
        assert np.array_equal(got[idx], qw_ref[k, n])


def _two_step(ops, lin, a_dev):
    """quant_act_per_token, then qgemm_w8a8_fp8 on its codes (the unfused path)."""
    qa, sa = ops.quantize_activations(a_dev)
    return lin(a_dev, qa=qa, sa=sa)


def _fp8_gemm(ops, a_bits, w_bits):
    fw = ops.Fp8Weight.from_bf16(dev_bf16(w_bits))
    lin = ops.W8A8Fp8Linear(fw)
    y = _two_step(ops, lin, dev_bf16(a_bits))
    torch.cuda.synchronize()
    return host_bits16(y)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (1280, 144), (1024, 272)])
@pytest.mark.parametrize("M", [1, 3, 4, 16, 17, 33, 64, 65, 100, 256, 300])
def test_fp8_gemm_parity(ops, M, K, N):
    announce(f"qgemm_w8a8_fp8 M={M} K={K} N={N}")
    w = synth.weights(K, N, seed=5 + K + N)
    a = synth.activations(M, K, seed=7 + M)
    qa, sa = f8.quant_act_per_token(a)
    qw, sw = f8.quant_weight_per_channel(w)
    y = _fp8_gemm(ops, a, w)
    assert_close_rms(y, f8.gemm_ref(qa, sa, qw, sw), what=f"fp8 M={M} K={K} N={N}")


_QW = {}


@pytest.mark.parametrize("B", [1, 16, 128, 512, 1024])
@pytest.mark.parametrize("j,name,K,N", [(1, "o", 4096, 4096), (3, "down", 14336, 4096)])
def test_fp8_gemm_llama3_8b_shapes(ops, B, j, name, K, N):
    announce(f"qgemm_w8a8_fp8 8B {name} B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(0, j))
    a = synth.activations(1024, K, seed=synth.activation_seed(0, j))[:B]
    y = _fp8_gemm(ops, a, w)
    rows = np.unique(np.random.default_rng(B).integers(0, B, 32))
    qa, sa = f8.quant_act_per_token(a[rows])
    if j not in _QW:                                   # the oracle's weight codes, once per shape
        _QW[j] = f8.quant_weight_per_channel(w)
    qw, sw = _QW[j]
    assert_close_rms(y[rows], f8.gemm_ref(qa, sa, qw, sw), what=f"fp8 {name} B={B}")


def test_fp8_all_ones_exact(ops):
    announce("qgemm_w8a8_fp8 all-ones")
    K, N = 4096, 32
    ones_w = f32_to_bf16_bits(np.ones((K, N), dtype=np.float32))
    for M in (2, 100):
        a = f32_to_bf16_bits(np.ones((M, K), dtype=np.float32))
        y = _fp8_gemm(ops, a, ones_w)
        yf = (y.astype(np.uint32) << 16).view(np.float32)
        assert np.all(yf == 4096.0)


@pytest.mark.parametrize("M", [4, 300])
def test_fp8_deterministic(ops, M):
    announce(f"qgemm_w8a8_fp8 determinism M={M}")
    K, N = 4096, 1024
    fw = ops.Fp8Weight.from_bf16(dev_bf16(synth.weights(K, N, seed=8)))
    lin = ops.W8A8Fp8Linear(fw)
    a = dev_bf16(synth.activations(M, K, seed=9))
    y1 = host_bits16(lin(a))
    y2 = host_bits16(lin(a))
    assert np.array_equal(y1, y2)


# (M, K, N, tiles, S): shapes whose tiles cannot fill 256 CUs, so K is split S
# ways: 64 x 128 tiles where 128-row tiles would fill at most a quarter of the
# CUs (M = 200, 100), 128 x 128 tiles at M = 300; N = 1040 leaves a ragged last
# column tile, S = 5 a partial group of four slots in the final reduction
@pytest.mark.parametrize("M,K,N,tiles,S", [(200, 14336, 4096, 128, 2), (100, 14336, 1040, 18, 8),
                                            (100, 10240, 1040, 18, 5), (300, 14336, 4096, 96, 4)])
def test_fp8_large_m_split_counters_reset(ops, M, K, N, tiles, S):
    """The K split writes unscaled fp32 slots and counts arrivals per tile (one
    32-bit counter each, in the counter region before the slots); the last
    arriver applies the scales.
    Every call leaves the counters at zero; repeated calls on one workspace are
    bit-identical and match the oracle."""
    announce(f"qgemm_w8a8_fp8 large-M split M={M} K={K} N={N}")
    nbytes = ops.w8a8_workspace_bytes(M, N, K)
    assert nbytes == 65536 + S * M * N * 4          # counter region, then S slots
    w = synth.weights(K, N, seed=83)
    a = synth.activations(M, K, seed=89)
    qa, sa = f8.quant_act_per_token(a)
    qw, sw = f8.quant_weight_per_channel(w)
    ref = f8.gemm_ref(qa, sa, qw, sw)
    lin = ops.W8A8Fp8Linear(ops.Fp8Weight.from_bf16(dev_bf16(w)))
    ad = dev_bf16(a)
    first = None
    for _ in range(3):
        y = host_bits16(_two_step(ops, lin, ad))
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(lin._ws[:65536])) == 0      # counters (first 4 * tiles bytes)
        assert_close_rms(y, ref, what=f"fp8 split M={M} K={K} N={N}")
        if first is None:
            first = y
        assert np.array_equal(y, first)


# ---------------------------------------------------------------- wide shapes

# Weights of the wide Llama-3-8B shapes, drawn on the device (torch's
# generator; both sides receive the same bits) and quantized once per shape;
# the oracle gets the bits of 256 sampled columns (per-channel quantization is
# exact on a column subset) and of up to 32 sampled rows.
_WIDE = {}
WIDE_SHAPES = [("qkv", 4096, 6144, 1000), ("gate_up", 4096, 28672, 1002), ("lm_head", 4096, 128256, 1128)]


def _wide(ops, name, K, N, seed):
    if name not in _WIDE:
        _WIDE.clear()                                   # one shape resident at a time
        w_dev = synth.normal_bf16_device((K, N), seed, synth.WEIGHT_STD, "cuda")
        cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(seed).integers(0, N, 254)]))
        w_cols = host_bits16(w_dev[:, torch.from_numpy(cols).cuda()])
        wt = ops.Fp8Weight.from_bf16(w_dev)
        del w_dev
        torch.cuda.synchronize()
        _WIDE[name] = (wt, cols, f8.quant_weight_per_channel(w_cols))
    return _WIDE[name]


@pytest.mark.parametrize("name,K,N,seed", WIDE_SHAPES)
@pytest.mark.parametrize("B", [1, 16, 128, 512, 1024])
def test_fp8_gemm_wide_shapes_sampled(ops, name, K, N, seed, B):
    kern = ops.w8a8_kernel_for(B, N, K)
    announce(f"qgemm_w8a8_fp8 8B {name} B={B} ({kern})")
    wt, cols, (qw, sw) = _wide(ops, name, K, N, seed)
    a = synth.activations(B, K, seed=seed + B)
    y = host_bits16(_two_step(ops, ops.W8A8Fp8Linear(wt), dev_bf16(a)))
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(B).integers(0, B, 32))
    qa, sa = f8.quant_act_per_token(a[rows])
    assert_close_rms(y[rows][:, cols], f8.gemm_ref(qa, sa, qw, sw), what=f"fp8 {name} B={B} {kern}")


def test_fp8_wide_shapes_cover_every_instantiation(ops):
    """The wide-shape cases above run the two-column-tile small-M kernel (CT = 2)
    and the 256-column large-M tiles (NB = 2) besides the narrow forms."""
    names = {ops.w8a8_kernel_for(B, N, K) for (_, K, N, _) in WIDE_SHAPES for B in (1, 16, 128, 512, 1024)}
    assert "w8a8_small_m_kernel<1, 2>" in names and "w8a8_small_m_kernel<1, 1>" in names, names
    large = [n for n in names if n.startswith("w8a8_large_m_kernel<")]
    assert any(n.split("<")[1].split(",")[1].strip() == "2" for n in large), names
    assert any(n.split("<")[1].split(",")[1].strip() == "1" for n in large), names
