"""GPU parity of the W4A16 path (pack, dequant, GEMM) against the CPU oracle.

Packing, codes and dequantized weights: bit-exact.  GEMM: max |err| <= 2e-2 x
RMS of the fp64 oracle output, per call.  Inputs are the seeded synthetic
draws of weight_only_quantized_w4a16_amd.synth; both sides receive the same bits.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16, host_u8, host_u32
from oracle import int4_g128 as q4
from oracle.bf16 import bf16_bits_to_f32, f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _pack(ops, w_bits):
    K, N = w_bits.shape
    wt = ops.Int4G128Weight.from_bf16(dev_bf16(w_bits))
    torch.cuda.synchronize()
    return wt


def _gemm(ops, wt, a_bits):
    lin = ops.W4A16Linear(wt)
    y = lin(dev_bf16(a_bits))
    torch.cuda.synchronize()
    return host_bits16(y)


# ---------------------------------------------------------------- packing

@pytest.mark.parametrize("K,N", [(128, 16), (384, 48), (1280, 144), (4096, 4096)])
def test_pack_bit_exact(ops, K, N):
    announce(f"pack_int4_g128 K={K} N={N} seed={K + N}")
    w = synth.weights(K, N, seed=K + N)
    codes, s = q4.quantize(w)
    packed_ref, scales_ref = q4.pack_native(codes, s)
    wt = _pack(ops, w)
    assert np.array_equal(host_u32(wt.packed), packed_ref)
    assert np.array_equal(host_bits16(wt.scales), scales_ref)


def _native_nibbles(packed, k, n, K):
    """Codes at (k, n) read from a native buffer by the layout formula."""
    G = K // 128
    nt, c = n // 16, n % 16
    g, r = k // 128, k % 128
    t, r = r // 32, r % 32
    j, i = r // 8, r % 8
    slot = np.where(i % 2 == 0, i // 2, 4 + i // 2)
    word = (nt * G + g) * 256 + (16 * j + c) * 4 + t
    return (packed[word] >> (4 * slot).astype(np.uint32)) & np.uint32(0xF)


@pytest.mark.parametrize("name,K,N", [("qkv", 4096, 6144), ("down", 14336, 4096),
                                      ("lm_head", 4096, 128256)])
def test_pack_full_shape_sampled(ops, name, K, N):
    announce(f"pack_int4_g128 full {name} K={K} N={N}")
    w = synth.weights(K, N, seed=77)
    wt = _pack(ops, w)
    packed = host_u32(wt.packed)
    scales = host_bits16(wt.scales)
    rng = np.random.default_rng(5)
    cols = np.unique(rng.integers(0, N, 64))
    codes, s = q4.quantize(w[:, cols])             # per-column quantization: exact on a subset
    kk = np.repeat(np.arange(K), cols.size)
    nn = np.tile(cols, K)
    got = _native_nibbles(packed, kk, nn, K).reshape(K, cols.size)
    assert np.array_equal(got, codes)
    G = K // 128
    sidx = ((cols[None, :] // 16) * G + np.arange(G)[:, None]) * 16 + cols[None, :] % 16
    assert np.array_equal(scales[sidx], s)


# ---------------------------------------------------------------- dequant

@pytest.mark.parametrize("K,N", [(128, 16), (1280, 144), (4096, 4096)])
def test_dequant_bit_exact(ops, K, N):
    announce(f"dequant_int4_g128 K={K} N={N}")
    w = synth.weights(K, N, seed=3 * K + N)
    codes, s = q4.quantize(w)
    wt = _pack(ops, w)
    wd, cd = wt.dequant(with_codes=True)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(cd), codes)
    assert np.array_equal(host_bits16(wd), q4.dequant_bf16_bits(codes, s))


def test_dequant_exhaustive_codes_and_scales(ops):
    """Every code 0..15 under every finite bf16 scale, through the GPU unpack."""
    announce("dequant_int4_g128 exhaustive codes x scales")
    s_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s_bits = s_bits[np.isfinite(bf16_bits_to_f32(s_bits))]
    N = s_bits.size // 16 * 16
    s_bits = s_bits[:N].reshape(1, N)
    K = 128
    codes = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))
    packed, scales = q4.pack_native(codes, s_bits)
    p_dev = torch.from_numpy(packed.view(np.int32)).cuda()
    s_dev = torch.from_numpy(scales.view(np.int16)).cuda()
    wd = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    cd = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    ops.dequant_int4_g128(p_dev, s_dev, K, N, wd, cd)
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(cd), codes)
    with np.errstate(over="ignore"):
        ref = q4.dequant_bf16_bits(codes, s_bits)
    assert np.array_equal(host_bits16(wd), ref)


# ---------------------------------------------------------------- GEMM

SMALL_SHAPES = [(128, 16), (256, 64), (1280, 144), (1024, 272)]
M_VALUES = [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, 48, 64, 65, 100, 128, 130, 256]


@pytest.mark.parametrize("K,N", SMALL_SHAPES)
@pytest.mark.parametrize("M", M_VALUES)
def test_gemm_parity(ops, M, K, N):
    announce(f"qgemm_w4a16 M={M} K={K} N={N}")
    w = synth.weights(K, N, seed=11 + K + N)
    a = synth.activations(M, K, seed=17 + M)
    codes, s = q4.quantize(w)
    y = _gemm(ops, _pack(ops, w), a)
    assert_close_rms(y, q4.gemm_ref(a, codes, s), what=f"M={M} K={K} N={N}")


def test_gemm_config1_single_gemm(ops):
    """Activations [4, 4096] ~ N(0,1) seed 1; weights [4096, 4096] std 0.02 seed 0."""
    announce("qgemm_w4a16 M=4 K=4096 N=4096 (single GEMM)")
    w = synth.weights(4096, 4096, seed=0)
    a = synth.activations(4, 4096, seed=1)
    codes, s = q4.quantize(w)
    y = _gemm(ops, _pack(ops, w), a)
    ref = q4.gemm_ref(a, codes, s)
    assert_close_rms(y, ref, what="single GEMM")
    # Beyond the final bf16 rounding (at most one bf16 ulp of |y|), the folded
    # form carries only fp32 accumulation error: far below 1e-3 of the RMS.
    got = bf16_bits_to_f32(y).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    assert np.all(np.abs(got - ref) <= ulp + 1e-3 * rms)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("j,name,K,N", [(0, "qkv", 4096, 6144), (1, "o", 4096, 4096),
                                        (2, "gate_up", 4096, 28672), (3, "down", 14336, 4096)])
def test_gemm_llama3_8b_layer_shapes(ops, B, j, name, K, N):
    announce(f"qgemm_w4a16 8B {name} B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(0, j))
    a = synth.activations(1024, K, seed=synth.activation_seed(0, j))[:B]
    codes, s = q4.quantize(w)
    y = _gemm(ops, _pack(ops, w), a)
    assert_close_rms(y, q4.gemm_ref(a, codes, s), what=f"{name} B={B}")


@pytest.mark.parametrize("B", [1, 16, 64, 256])
def test_gemm_llama3_8b_lm_head_sampled(ops, B):
    K, N = 4096, 128256
    announce(f"qgemm_w4a16 8B lm_head B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(32, 0))
    a = synth.activations(B, K, seed=synth.activation_seed(32, 0))
    y = _gemm(ops, _pack(ops, w), a)
    cols = np.unique(np.random.default_rng(B).integers(0, N, 512))
    codes, s = q4.quantize(w[:, cols])
    assert_close_rms(y[:, cols], q4.gemm_ref(a, codes, s), what=f"lm_head B={B}")


_W70 = {}


def _w70(ops, j, K, N):
    """Llama-3-70B layer weights (and their packed form), generated once per shape."""
    if j not in _W70:
        w = synth.weights(K, N, seed=synth.weight_seed(100, j))
        _W70[j] = (w, _pack(ops, w))
    return _W70[j]


@pytest.mark.parametrize("B", [1, 8, 16, 64, 256])
@pytest.mark.parametrize("j,name,K,N", [(0, "qkv", 8192, 10240), (1, "o", 8192, 8192),
                                        (2, "gate_up", 8192, 57344), (3, "down", 28672, 8192)])
def test_gemm_llama3_70b_layer_shapes_sampled(ops, B, j, name, K, N):
    """70B layer shapes at the batches of the 70B workload; 256 sampled output
    columns against the oracle (per-column quantization is exact on a subset)."""
    announce(f"qgemm_w4a16 70B {name} B={B}")
    w, wt = _w70(ops, j, K, N)
    a = synth.activations(B, K, seed=synth.activation_seed(100, j) + B)
    y = _gemm(ops, wt, a)
    cols = np.unique(np.random.default_rng(1000 + B).integers(0, N, 256))
    codes, s = q4.quantize(w[:, cols])
    assert_close_rms(y[:, cols], q4.gemm_ref(a, codes, s), what=f"70B {name} B={B}")


@pytest.mark.parametrize("B", [1, 8, 16, 64, 256])
def test_gemm_llama3_70b_lm_head_sampled(ops, B):
    """The 70B LM head 8192 -> 128256 (whole-K decode workgroups at B <= 8, a
    decode K split at B = 16, large-M tiles at 64 / 256): weights drawn on the device by torch's generator, 256
    sampled columns and up to 40 sampled rows against the oracle."""
    K, N = 8192, 128256
    global _W70_HEAD
    if _W70_HEAD is None:
        w_dev = synth.normal_bf16_device((K, N), synth.weight_seed(180, 0), synth.WEIGHT_STD, "cuda")
        cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(7).integers(0, N, 254)]))
        w_cols = host_bits16(w_dev[:, torch.from_numpy(cols).cuda()])
        wt = ops.Int4G128Weight.from_bf16(w_dev)
        del w_dev
        torch.cuda.synchronize()
        _W70_HEAD = (wt, cols, q4.quantize(w_cols))
    wt, cols, (codes, s) = _W70_HEAD
    kern = ops.w4a16_kernel_for(B, N, K)
    announce(f"qgemm_w4a16 70B lm_head B={B} ({kern})")
    a = synth.activations(B, K, seed=synth.activation_seed(180, 0) + B)
    y = _gemm(ops, wt, a)
    rows = np.unique(np.random.default_rng(B).integers(0, B, 40))
    assert_close_rms(y[rows][:, cols], q4.gemm_ref(a[rows], codes, s), what=f"70B lm_head B={B} {kern}")


_W70_HEAD = None


# B spans the small-M kernels (17..64 rows where the large-M grid would not
# cover the CUs), 64-row large-M tiles (M <= 64, 128-row tiles filling at most
# half of the CUs, and gate_up at 570 / 576 rows where 64 x 256 tiles take
# fewer launch rounds; 570 leaves a ragged last tile) and 128-row tiles; at
# 272 and 300 the last row tile has 16 / 44 rows, so its second row of waves
# has none (those waves only copy); the last rows are always among the checked
@pytest.mark.parametrize("B", [24, 32, 48, 64, 96, 128, 192, 256, 272, 300, 512, 570, 576, 1024])
@pytest.mark.parametrize("j,name,K,N", [(0, "qkv", 4096, 6144), (1, "o", 4096, 4096),
                                        (2, "gate_up", 4096, 28672), (3, "down", 14336, 4096)])
def test_gemm_large_batch_sampled_rows(ops, B, j, name, K, N):
    announce(f"qgemm_w4a16 8B {name} B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(0, j))
    a = synth.activations(1024, K, seed=synth.activation_seed(0, j))[:B]
    codes, s = q4.quantize(w)
    y = _gemm(ops, _pack(ops, w), a)
    rows = np.unique(np.concatenate([np.random.default_rng(B).integers(0, B, 48), np.arange(max(0, B - 4), B)]))
    assert_close_rms(y[rows], q4.gemm_ref(a[rows], codes, s), what=f"{name} B={B}")


def test_gemm_identity_weight(ops):
    """W = I: the oracle gives 0.998046875 * a exactly; the folded kernel must land
    within one bf16 ulp of it element by element, plus the fp32 rounding of its
    -136 * sum(a) offset term (a cancellation on small outputs)."""
    announce("qgemm_w4a16 identity")
    K = N = 512
    w = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    codes, s = q4.quantize(w)
    for M in (4, 200):
        a = synth.activations(M, K, seed=23)
        y = _gemm(ops, _pack(ops, w), a)
        ref = q4.gemm_ref(a, codes, s)
        assert np.array_equal(ref, 0.998046875 * bf16_bits_to_f32(a).astype(np.float64))
        assert_close_rms(y, ref, what=f"identity M={M}")
        got = bf16_bits_to_f32(y).astype(np.float64)
        # one bf16 ulp, plus the fp32 cancellation of the offset term:
        # 136 * sum over the row's group of |a|, at a few fp32 ulps, times the scale
        af = np.abs(bf16_bits_to_f32(a).astype(np.float64)).reshape(M, K // 128, 128).sum(axis=2)
        cancel = np.repeat(af, 128, axis=1) * 136 * 0.142578125 * 2.0 ** -20
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + cancel)


def test_gemm_all_ones(ops):
    """All-ones a and W, K = 4096: Y64 = 4088, and bf16(4088) = 4096 (a tie to even)."""
    announce("qgemm_w4a16 all-ones")
    K, N = 4096, 64
    w = f32_to_bf16_bits(np.ones((K, N), dtype=np.float32))
    for M in (3, 100):
        a = f32_to_bf16_bits(np.ones((M, K), dtype=np.float32))
        y = _gemm(ops, _pack(ops, w), a)
        assert np.all(bf16_bits_to_f32(y) == 4096.0)


def test_gemm_zero_weight_and_zero_rows(ops):
    announce("qgemm_w4a16 zero weight / zero rows")
    K, N = 512, 32
    w = np.zeros((K, N), dtype=np.uint16)
    a = synth.activations(5, K, seed=2)
    assert np.all(_gemm(ops, _pack(ops, w), a) == 0)
    w = synth.weights(K, N, seed=3)
    a[2] = 0
    y = _gemm(ops, _pack(ops, w), a)
    assert np.all(bf16_bits_to_f32(y[2]) == 0)


def test_gemm_m_zero_launches_nothing(ops):
    announce("qgemm_w4a16 M=0")
    wt = _pack(ops, synth.weights(128, 16, seed=1))
    y = torch.full((1, 16), 7.0, dtype=torch.bfloat16, device="cuda")
    a = torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda")
    ops.qgemm_w4a16(a, wt.packed, wt.scales, y, 0, 16, 128)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("M", [4, 300])
def test_gemm_deterministic(ops, M):
    announce(f"qgemm_w4a16 determinism M={M}")
    K, N = 4096, 1024
    wt = _pack(ops, synth.weights(K, N, seed=8))
    a = dev_bf16(synth.activations(M, K, seed=9))
    lin = ops.W4A16Linear(wt)
    y1 = host_bits16(lin(a))
    y2 = host_bits16(lin(a))
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M", [1, 3, 5, 16])
@pytest.mark.parametrize("K,N", [(1024, 9600), (2048, 8208), (1280, 8192), (8320, 144), (8192, 2064)])
def test_gemm_wide_small_m(ops, M, K, N):
    """Small M through the decode kernel: wide outputs in one K-slice (tile ranges
    that do not divide evenly over workgroups and waves), long-K narrow outputs
    split across workgroups (M > 4), the rest through the split-K kernel."""
    announce(f"qgemm_w4a16 wide M={M} K={K} N={N}")
    w = synth.weights(K, N, seed=31 + K + N)
    a = synth.activations(M, K, seed=37 + M)
    codes, s = q4.quantize(w)
    y = _gemm(ops, _pack(ops, w), a)
    assert_close_rms(y, q4.gemm_ref(a, codes, s), what=f"wide M={M} K={K} N={N}")


# from 9 rows (up to 8 the small-M kernel runs these shapes without a workspace)
@pytest.mark.parametrize("M,K,N", [(9, 14336, 4096), (16, 14336, 4096), (16, 8320, 144)])
def test_decode_workspace_counters_reset(ops, M, K, N):
    """Decode shapes whose activation slice does not fit in LDS split K across
    workgroups and count arrivals in the workspace: the 64 KiB counter region
    (one 32-bit counter per column strip, at most N/16 of them), then S slots
    of N/16 fp32 tiles.  Every call resets its counters, so repeated calls on
    one workspace keep giving the right answer and the counter region reads
    zero after each call."""
    announce(f"qgemm_w4a16 workspace counters M={M} K={K} N={N}")
    nbytes = ops.w4a16_workspace_bytes(M, N, K)
    nt = N // 16
    assert nbytes > 65536 and (nbytes - 65536) % (nt * 1024) == 0
    assert (nbytes - 65536) // (nt * 1024) >= 2
    w = synth.weights(K, N, seed=41)
    a = synth.activations(M, K, seed=43)
    codes, s = q4.quantize(w)
    lin = ops.W4A16Linear(_pack(ops, w))
    ad = dev_bf16(a)
    first = None
    for _ in range(3):
        y = host_bits16(lin(ad))
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(lin._ws[:65536])) == 0
        assert_close_rms(y, q4.gemm_ref(a, codes, s), what=f"M={M} K={K} N={N}")
        if first is None:
            first = y
        assert np.array_equal(y, first)


# tiles: output tiles these shapes use (too few for 256 CUs, so K is split):
# 64 x 128 tiles at M = 200 (4 x 32) and M = 48 (1 x 32), 128 x 128 tiles at
# M = 384, N = 8192 (3 x 64)
@pytest.mark.parametrize("M,K,N,tiles", [(200, 14336, 4096, 128), (48, 14336, 4096, 32),
                                          (384, 28672, 8192, 192)])
def test_large_m_split_counters_reset(ops, M, K, N, tiles):
    """Large-M shapes whose tiles cannot fill the GPU split K across workgroups
    and count arrivals per tile (one 32-bit counter each, in the 64 KiB
    counter region at the front of the workspace); every call leaves those
    counters at zero, and repeated calls on one workspace are bit-identical and
    match the oracle."""
    announce(f"qgemm_w4a16 large-M split M={M} K={K} N={N}")
    assert ops.w4a16_kernel_for(M, N, K).startswith("w4a16_large_m_kernel<")
    w = synth.weights(K, N, seed=47)
    a = synth.activations(M, K, seed=53)
    codes, s = q4.quantize(w)
    lin = ops.W4A16Linear(_pack(ops, w))
    ad = dev_bf16(a)
    ref = q4.gemm_ref(a, codes, s)
    first = None
    for _ in range(3):
        y = host_bits16(lin(ad))
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(lin._ws[:4 * tiles])) == 0    # the tile counters
        assert int(torch.count_nonzero(lin._ws[:65536])) == 0
        assert_close_rms(y, ref, what=f"M={M} K={K} N={N}")
        if first is None:
            first = y
        assert np.array_equal(y, first)
