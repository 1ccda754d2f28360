"""qgemm_w4a8_fp8_grouped_dynamic: bf16 routed rows in, the per-token e4m3
quantization inside the call.  Its output equals quant_act_per_token followed
by qgemm_w4a8_fp8_grouped bit for bit, whether each workgroup quantizes its
item's rows in LDS (few rows per expert) or the codes go through the workspace
(the large-tile path, long rows): Qwen3-30B-A3B expert shapes over the routed
batches of a decode step, ragged expert sizes, rows that reach every branch of
the quantization (zero, large, tiny and subnormal rows, exact code ties), one
workspace serving fused and unfused calls in turn; sampled experts are also
checked against the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
from oracle import fp8_e4m3 as f8
from oracle import int4_g128 as q4
from oracle import w4a8
from oracle.bf16 import f32_to_bf16_bits
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _rows(T, K, seed):
    """N(0, 1) routed rows with the special rows spread over the first experts."""
    f = (synth.normal_bf16((T, K), seed).astype(np.uint32) << 16).view(np.float32).copy()
    rng = np.random.default_rng(seed)
    special = [np.zeros(K, np.float32),
               rng.standard_normal(K).astype(np.float32) * np.float32(1e30),
               rng.standard_normal(K).astype(np.float32) * np.float32(1e-33),
               rng.standard_normal(K).astype(np.float32) * np.float32(1e-39),
               np.resize(np.array([448.0, 1.0625, 1.1875, -2.125, 0.5, 1.5, -2.5, 3.0], np.float32), K)]
    for j, row in enumerate(special):
        if 2 * j + 1 < T:
            f[2 * j + 1] = row
    return f32_to_bf16_bits(f)


def _both(ops, gw, a_bits, offsets):
    a = dev_bf16(a_bits)
    off = torch.from_numpy(offsets).cuda()
    qa, sa = ops.quantize_activations(a)
    y_two = host_bits16(gw.w4a8(qa, sa, off))
    y_dyn = host_bits16(gw.w4a8_dynamic(a, off))
    torch.cuda.synchronize()
    return y_two, y_dyn


_GW = {}


def _qwen3_weight(ops, j):
    if j not in _GW:
        E = synth.QWEN3_MOE_EXPERTS
        _, K, N = synth.QWEN3_MOE_SHAPES[j]
        w = synth.normal_bf16_device((E, K, N), seed=177 + j, std=synth.WEIGHT_STD, device="cuda")
        _GW[j] = (ops.GroupedInt4Weight.from_bf16(w), w)
    return _GW[j]


@pytest.mark.parametrize("j", [0, 1])
@pytest.mark.parametrize("B", [1, 2, 5, 16, 40, 64, 256])
def test_qwen3_dynamic_equals_two_calls(ops, B, j):
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    name, K, N = synth.QWEN3_MOE_SHAPES[j]
    T = B * k
    kern = ops.w4a8_grouped_dynamic_kernel_for(E, T, N, K)
    announce(f"qgemm_w4a8_fp8_grouped_dynamic qwen3 {name} B={B} ({kern})")
    _, offsets = synth.moe_routing(B, E, k, seed=B)
    gw, w = _qwen3_weight(ops, j)
    a = _rows(T, K, seed=31 + B)
    y_two, y_dyn = _both(ops, gw, a, offsets)
    assert np.array_equal(y_dyn, y_two), f"{name} B={B} {kern}"
    if B in (1, 16):
        qa, sa = f8.quant_act_per_token(a)
        nonempty = [e for e in range(E) if offsets[e + 1] > offsets[e]]
        for e in nonempty[:: max(1, len(nonempty) // 4)]:
            r0, r1 = offsets[e], offsets[e + 1]
            ref = w4a8.grouped_gemm_ref(qa, sa, offsets, {e: q4.quantize(host_bits16(w[e]))})[e]
            for r in range(r0, r1):                      # each row against its own output scale
                if np.max(np.abs(ref[r - r0])) > 1e-30:
                    assert_close_rms(y_dyn[r:r + 1], ref[r - r0:r - r0 + 1], what=f"{name} B={B} row {r}")


@pytest.mark.parametrize("sizes,K,N", [([0, 1, 17, 0, 3, 5], 256, 64), ([2, 0, 0, 5, 1, 0, 3, 0, 0, 4], 384, 48),
                                       ([40, 0, 5], 1024, 272), ([0, 20, 25, 0], 2048, 64),
                                       ([0, 9, 33, 0, 16, 7], 1024, 272), ([0, 65, 33, 0, 128, 7, 70], 640, 272),
                                       ([1, 2, 3], 4096, 64), ([7], 512, 64), ([300], 256, 272)])
def test_ragged_dynamic_equals_two_calls(ops, sizes, K, N):
    """Fused items of 1..16 rows and of up to 32 rows (an expert of 40 rows in two
    items), then unfused: 65 routed rows, the large tile, rows of 4096; a single
    expert with few rows (fused) and with 300 (the large tile)."""
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(offsets[-1])
    E = len(sizes)
    kern = ops.w4a8_grouped_dynamic_kernel_for(E, T, N, K)
    announce(f"qgemm_w4a8_fp8_grouped_dynamic sizes={sizes} K={K} N={N} ({kern})")
    w = torch.stack([dev_bf16(synth.weights(K, N, seed=600 + e)) for e in range(E)])
    gw = ops.GroupedInt4Weight.from_bf16(w)
    y_two, y_dyn = _both(ops, gw, _rows(T, K, seed=T + K), offsets)
    assert np.array_equal(y_dyn, y_two), f"sizes={sizes} K={K} N={N} {kern}"


def test_fused_where_expected(ops):
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    fused = lambda T, K, N: ops.w4a8_grouped_dynamic_kernel_for(E, T, N, K) == "w4a8_grouped_dyn_kernel"
    for _, K, N in synth.QWEN3_MOE_SHAPES:
        assert fused(1 * k, K, N) and fused(5 * k, K, N)
        assert not fused(6 * k, K, N) and not fused(16 * k, K, N)
        assert not fused(1024 * k, K, N)                 # the large tile
    assert not fused(8, 4096, 64)                        # rows longer than 2048
    assert ops.w4a8_grouped_dynamic_workspace_bytes(E, 8, 1536, 2048) == 0     # fused: none
    assert ops.w4a8_grouped_dynamic_workspace_bytes(E, 128, 1536, 2048) >= 128 * 2048


def test_one_workspace_fused_and_unfused(ops):
    """One grouped weight object: a fused call, an unfused (large tile) call
    whose codes go through the workspace, then fused again."""
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    gw, _ = _qwen3_weight(ops, 0)
    _, K, N = synth.QWEN3_MOE_SHAPES[0]
    announce("qgemm_w4a8_fp8_grouped_dynamic workspace across fused and unfused calls")
    for B in (4, 512, 4, 512):
        T = B * k
        _, offsets = synth.moe_routing(B, E, k, seed=B + 1)
        y_two, y_dyn = _both(ops, gw, _rows(T, K, seed=B), offsets)
        assert np.array_equal(y_dyn, y_two), B
