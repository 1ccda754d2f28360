"""GPU parity of qgemm_w4a16_grouped (expert-grouped W4A16) against the oracle.

Each expert's output rows: max |err| <= 2e-2 x RMS of that expert's fp64
oracle rows.  Covers ragged and empty experts, the three row-chunk sizes,
one expert owning every row, the Qwen3-30B-A3B expert shapes with 128 experts
under seeded top-8 routing, repeat determinism, and malformed offsets staying
inside the output."""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
from oracle import int4_g128 as q4
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _run(ops, w_list, a_bits, offsets):
    E = len(w_list)
    K, N = w_list[0].shape
    w = torch.stack([dev_bf16(x) for x in w_list])
    gw = ops.GroupedInt4Weight.from_bf16(w)
    y = gw(dev_bf16(a_bits), torch.from_numpy(np.asarray(offsets, np.int32)).cuda())
    torch.cuda.synchronize()
    return host_bits16(y), gw


def _check(y, a_bits, offsets, w_list, experts=None):
    for e in (range(len(w_list)) if experts is None else experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        ref = q4.grouped_gemm_ref(a_bits, offsets, {e: q4.quantize(w_list[e])})[e]
        assert_close_rms(y[r0:r1], ref, what=f"expert {e} rows {r0}:{r1}")


@pytest.mark.parametrize("sizes,K,N", [
    ([0, 1, 17, 0, 40, 3, 70, 5], 256, 64),          # mean 17 rows -> 32-row chunks
    ([2, 0, 0, 5, 1, 0, 3, 0, 0, 4], 384, 48),        # mean <= 16 -> 16-row chunks
    ([90, 33, 0, 65, 128], 128, 16),                   # mean > 32 -> 128-row large-M items
    ([0, 0, 200, 0], 512, 272),                        # one expert owns every row (large-M)
    ([300, 0, 129, 40, 7], 1024, 1040),                # large-M: multi-chunk expert, ragged N
])
def test_grouped_ragged(ops, sizes, K, N):
    announce(f"qgemm_w4a16_grouped sizes={sizes} K={K} N={N}")
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(offsets[-1])
    w_list = [synth.weights(K, N, seed=100 + e) for e in range(len(sizes))]
    a = synth.activations(T, K, seed=T + K)
    y, _ = _run(ops, w_list, a, offsets)
    _check(y, a, offsets, w_list)


@pytest.mark.parametrize("B", [1, 16, 64, 256, 1024])
@pytest.mark.parametrize("name,K,N", synth.QWEN3_MOE_SHAPES)
def test_grouped_qwen3_moe_shapes(ops, B, name, K, N):
    """128 experts of the real shape, seeded top-8 routing of B tokens; the
    weights are drawn on the device and the checked experts' bf16 bits copied
    back for the oracle."""
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    announce(f"qgemm_w4a16_grouped qwen3 {name} B={B} E={E} K={K} N={N}")
    token, offsets = synth.moe_routing(B, E, k, seed=B)
    T = B * k
    x = synth.activations(B, K, seed=7 + B)
    a = x[token]                                       # rows grouped by expert
    w = synth.normal_bf16_device((E, K, N), seed=55, std=synth.WEIGHT_STD, device="cuda")
    gw = ops.GroupedInt4Weight.from_bf16(w)
    y = host_bits16(gw(dev_bf16(a), torch.from_numpy(offsets).cuda()))
    nonempty = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    check = nonempty[:: max(1, len(nonempty) // 6)] + [nonempty[-1]]
    w_host = {e: host_bits16(w[e]) for e in check}
    for e in check:
        r0, r1 = offsets[e], offsets[e + 1]
        ref = q4.grouped_gemm_ref(a, offsets, {e: q4.quantize(w_host[e])})[e]
        assert_close_rms(y[r0:r1], ref, what=f"{name} B={B} expert {e}")
    assert T == offsets[-1]


def test_grouped_deterministic_and_reused_workspace(ops):
    announce("qgemm_w4a16_grouped determinism")
    sizes = [3, 0, 20, 9]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    w_list = [synth.weights(256, 32, seed=200 + e) for e in range(4)]
    a = synth.activations(32, 256, seed=5)
    y1, gw = _run(ops, w_list, a, offsets)
    off = torch.from_numpy(offsets).cuda()
    y2 = host_bits16(gw(dev_bf16(a), off))
    assert np.array_equal(y1, y2)
    # a smaller call on the same workspace, then the first again
    y3 = host_bits16(gw(dev_bf16(a[:3]), torch.tensor([0, 3, 3, 3, 3], dtype=torch.int32).cuda()))
    _check(y3, a[:3], np.array([0, 3, 3, 3, 3]), w_list)
    assert np.array_equal(host_bits16(gw(dev_bf16(a), off)), y1)


def test_grouped_malformed_offsets_stay_in_bounds(ops):
    """Offsets past T, decreasing and negative: the call completes and writes
    nothing outside the T output rows (a guard region after them stays put)."""
    announce("qgemm_w4a16_grouped malformed offsets")
    K, N, T = 256, 32, 24
    w_list = [synth.weights(K, N, seed=300 + e) for e in range(4)]
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(x) for x in w_list]))
    a = dev_bf16(synth.activations(T, K, seed=6))
    y = torch.full((T + 8, N), 7.0, dtype=torch.bfloat16, device="cuda")
    # clamped per expert: e0 [0, 24), e1 [24, 24), e2 [10, 10), e3 [3, 3)
    bad = torch.tensor([-5, 1 << 30, 10, 3, 3], dtype=torch.int32, device="cuda")
    gw(a, bad, out=y[:T])
    torch.cuda.synchronize()
    assert torch.all(y[T:] == 7.0)
    # expert 0 owns [0, 24) after clamping: its rows are well defined
    _check(host_bits16(y[:T]), synth.activations(T, K, seed=6), np.array([0, T, T, T, T]), w_list, [0])
