"""GPU parity of the W8A8-INT8 path against the CPU oracle.

Activation codes and scales, weight codes (native order) and scales:
bit-exact.  GEMM: max |err| <= 2e-2 x RMS of the fp64 oracle output (the
integer sum is exact on both sides; only the fp32 scaling and the bf16
rounding differ)."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16, host_u8
from oracle import fp8_e4m3 as f8
from oracle import int8 as i8
from oracle.bf16 import f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


# K spans every launch form: one wave per row (K <= 2048, 4096, 8192), one
# workgroup per row (14336, 28672) and the two-pass kernel for longer rows
@pytest.mark.parametrize("M,K", [(1, 128), (4, 4096), (16, 14336), (37, 1000), (256, 4096), (3, 8192),
                                 (5, 28672), (2, 40960)])
def test_act_quant_bit_exact(ops, M, K):
    announce(f"quant_act_per_token_int8 M={M} K={K}")
    a = synth.activations(M, K, seed=M + 2 * K)
    q, s = ops.quantize_activations_int8(dev_bf16(a))
    torch.cuda.synchronize()
    q_ref, s_ref = i8.quant_act_per_token(a)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_act_quant_every_code_and_ties(ops):
    announce("quant_act_per_token_int8 every code, ties, zero row")
    ints = np.arange(-127, 128, dtype=np.float32)
    mids = np.arange(-127, 127, dtype=np.float32) + 0.5
    row = np.zeros(512, dtype=np.float32)
    row[:255] = ints
    row[255:509] = mids
    a = f32_to_bf16_bits(np.stack([row, np.zeros(512, np.float32), row * np.float32(1e-3)]))
    q, s = ops.quantize_activations_int8(dev_bf16(a))
    torch.cuda.synchronize()
    q_ref, s_ref = i8.quant_act_per_token(a)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("K,N", [(128, 16), (384, 48), (4096, 4096)])
def test_weight_quant_bit_exact(ops, K, N):
    announce(f"quant_weight_int8_per_channel K={K} N={N}")
    w = synth.weights(K, N, seed=K * 5 + N)
    iw = ops.Int8Weight.from_bf16(dev_bf16(w))
    torch.cuda.synchronize()
    qw_ref, sw_ref = i8.quant_weight_per_channel(w)
    assert np.array_equal(iw.scales.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    assert np.array_equal(host_u8(iw.codes), f8.pack_native(qw_ref.view(np.uint8)))


def _two_step(ops, lin, a_dev):
    """quant_act_per_token_int8, then qgemm_w8a8_int8 on its codes (the unfused path)."""
    qa, sa = ops.quantize_activations_int8(a_dev)
    return lin(a_dev, qa=qa, sa=sa)


def _int8_gemm(ops, a_bits, w_bits):
    lin = ops.W8A8Int8Linear(ops.Int8Weight.from_bf16(dev_bf16(w_bits)))
    y = _two_step(ops, lin, dev_bf16(a_bits))
    torch.cuda.synchronize()
    return host_bits16(y)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 64), (1280, 144), (1024, 272)])
@pytest.mark.parametrize("M", [1, 3, 16, 17, 33, 64, 65, 100, 256, 300])
def test_int8_gemm_parity(ops, M, K, N):
    announce(f"qgemm_w8a8_int8 M={M} K={K} N={N}")
    w = synth.weights(K, N, seed=11 + K + N)
    a = synth.activations(M, K, seed=13 + M)
    qa, sa = i8.quant_act_per_token(a)
    qw, sw = i8.quant_weight_per_channel(w)
    y = _int8_gemm(ops, a, w)
    assert_close_rms(y, i8.gemm_ref(qa, sa, qw, sw), what=f"int8 M={M} K={K} N={N}")


_QW = {}


@pytest.mark.parametrize("B", [1, 16, 128, 512, 1024])
@pytest.mark.parametrize("j,name,K,N", [(1, "o", 4096, 4096), (3, "down", 14336, 4096)])
def test_int8_gemm_llama3_8b_shapes(ops, B, j, name, K, N):
    announce(f"qgemm_w8a8_int8 8B {name} B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(0, j))
    a = synth.activations(1024, K, seed=synth.activation_seed(0, j))[:B]
    y = _int8_gemm(ops, a, w)
    rows = np.unique(np.random.default_rng(B).integers(0, B, 32))
    qa, sa = i8.quant_act_per_token(a[rows])
    if j not in _QW:                                   # the oracle's weight codes, once per shape
        _QW[j] = i8.quant_weight_per_channel(w)
    qw, sw = _QW[j]
    assert_close_rms(y[rows], i8.gemm_ref(qa, sa, qw, sw), what=f"int8 {name} B={B}")


def test_int8_exact_integer_sums(ops):
    """Weights and activations that quantize to exact small integers make the
    integer sum the whole answer: all-ones gives 127^2 K exactly, scaled back
    to K; a +-1 pattern gives the signed count."""
    announce("qgemm_w8a8_int8 exact sums")
    K, N = 4096, 32
    for M in (2, 100):
        a = f32_to_bf16_bits(np.ones((M, K), dtype=np.float32))
        y = _int8_gemm(ops, a, f32_to_bf16_bits(np.ones((K, N), dtype=np.float32)))
        yf = (y.astype(np.uint32) << 16).view(np.float32)
        assert np.all(yf == 4096.0)


# 64 x 128 tiles (128-row tiles would fill at most a quarter of the CUs), K split S ways
@pytest.mark.parametrize("M,K,N,tiles,S", [(200, 14336, 4096, 128, 2), (100, 10240, 1040, 18, 5)])
def test_int8_large_m_split_counters_reset(ops, M, K, N, tiles, S):
    announce(f"qgemm_w8a8_int8 large-M split M={M} K={K} N={N}")
    nbytes = ops.w8a8_int8_workspace_bytes(M, N, K)
    assert nbytes == 65536 + S * M * N * 4          # counter region, then S slots
    w = synth.weights(K, N, seed=97)
    a = synth.activations(M, K, seed=101)
    qa, sa = i8.quant_act_per_token(a)
    qw, sw = i8.quant_weight_per_channel(w)
    ref = i8.gemm_ref(qa, sa, qw, sw)
    lin = ops.W8A8Int8Linear(ops.Int8Weight.from_bf16(dev_bf16(w)))
    ad = dev_bf16(a)
    first = None
    for _ in range(3):
        y = host_bits16(_two_step(ops, lin, ad))
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(lin._ws[:65536])) == 0      # counters (first 4 * tiles bytes)
        assert_close_rms(y, ref, what=f"int8 split M={M} K={K} N={N}")
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
        wt = ops.Int8Weight.from_bf16(w_dev)
        del w_dev
        torch.cuda.synchronize()
        _WIDE[name] = (wt, cols, i8.quant_weight_per_channel(w_cols))
    return _WIDE[name]


@pytest.mark.parametrize("name,K,N,seed", WIDE_SHAPES)
@pytest.mark.parametrize("B", [1, 16, 128, 512, 1024])
def test_int8_gemm_wide_shapes_sampled(ops, name, K, N, seed, B):
    kern = ops.w8a8_kernel_for(B, N, K)
    announce(f"qgemm_w8a8_int8 8B {name} B={B} ({kern})")
    wt, cols, (qw, sw) = _wide(ops, name, K, N, seed)
    a = synth.activations(B, K, seed=seed + B)
    y = host_bits16(_two_step(ops, ops.W8A8Int8Linear(wt), dev_bf16(a)))
    torch.cuda.synchronize()
    rows = np.unique(np.random.default_rng(B).integers(0, B, 32))
    qa, sa = i8.quant_act_per_token(a[rows])
    assert_close_rms(y[rows][:, cols], i8.gemm_ref(qa, sa, qw, sw), what=f"int8 {name} B={B} {kern}")


def test_int8_wide_shapes_cover_every_instantiation(ops):
    """The wide-shape cases above run the two-column-tile small-M kernel (CT = 2)
    and the 256-column large-M tiles (NB = 2) besides the narrow forms."""
    names = {ops.w8a8_kernel_for(B, N, K) for (_, K, N, _) in WIDE_SHAPES for B in (1, 16, 128, 512, 1024)}
    assert "w8a8_small_m_kernel<1, 2>" in names and "w8a8_small_m_kernel<1, 1>" in names, names
    large = [n for n in names if n.startswith("w8a8_large_m_kernel<")]
    assert any(n.split("<")[1].split(",")[1].strip() == "2" for n in large), names
    assert any(n.split("<")[1].split(",")[1].strip() == "1" for n in large), names
