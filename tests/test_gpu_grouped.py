"""GPU parity of qgemm_w4a16_grouped (expert-grouped W4A16) against the oracle.

Each expert's output rows: max |err| <= 2e-2 x RMS of that expert's fp64
oracle rows.  Covers ragged and empty experts, the three row-chunk sizes,
one expert owning every row, up to 1000 experts (several per lane of the
in-kernel work-item derivation), the Qwen3-30B-A3B expert shapes with 128
experts under seeded top-8 routing, repeat determinism, and malformed offsets
(clamped, or overlapping so that items past the grid's bound are dropped)
staying inside the output."""
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
    ([2, 0, 0, 5, 1, 0, 3, 0, 0, 4], 384, 48),        # mean <= 12 -> 16-row chunks
    ([13, 0, 20, 13, 19], 256, 64),                    # mean 13 -> 32-row chunks (every expert one item)
    ([31, 0, 60, 29, 30], 256, 1040),                  # mean 30 -> 64-row large-M items, 29..31 rows: half idle
    ([31, 0, 45, 20, 29], 256, 1040),                  # mean 25 -> 32-row chunks on the small tiles
    ([100, 60, 0], 384, 272),                          # mean 54 -> 64-row items on 64 x 128 tiles, ragged N
    ([160, 60, 0], 384, 272),                          # mean 74 -> 128-row items; 60 / 32 rows: second half idle
    ([90, 33, 0, 65, 128], 128, 16),                   # mean 79 -> 128-row large-M items
    ([0, 0, 200, 0], 512, 272),                        # one expert owns every row (large-M)
    ([5], 256, 48),                                    # a single expert, few rows
    ([300], 256, 272),                                 # a single expert, 128-row items (last one 44 rows)
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


def skewed_sizes(E, T, seed):
    """T routed rows over E experts: a skewed share per expert, about a third
    of the experts without rows."""
    rng = np.random.default_rng(seed)
    p = rng.random(E) ** 3
    p[rng.random(E) < 0.3] = 0.0
    p[rng.integers(E)] += 1e-3
    return rng.multinomial(T, p / p.sum())


# E = 1000: 16 experts per lane of the work-item derivation; E = 300 and 65:
# the last lanes partly or wholly empty; 16-row items, then the large tile
@pytest.mark.parametrize("E,T,K,N", [(1000, 600, 128, 16), (300, 2000, 128, 32), (65, 64, 256, 64),
                                     (300, 12000, 128, 272)])
def test_grouped_many_experts(ops, E, T, K, N):
    announce(f"qgemm_w4a16_grouped many experts E={E} T={T} K={K} N={N}")
    sizes = skewed_sizes(E, T, seed=E + T)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    w_list = [synth.weights(K, N, seed=1000 + e) for e in range(E)]
    a = synth.activations(T, K, seed=E)
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(x) for x in w_list]))
    y_dev = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda")
    gw(dev_bf16(a), torch.from_numpy(offsets).cuda(), out=y_dev)
    y = host_bits16(y_dev)
    assert not np.any(np.all(y == 0x40e0, axis=1)), "rows left unwritten"
    nonempty = [e for e in range(E) if sizes[e] > 0]
    _check(y, a, offsets, w_list, nonempty[:: max(1, len(nonempty) // 8)] + [nonempty[-1]])


@pytest.mark.parametrize("B", [1, 2, 4, 5, 16, 64, 256, 1024])
@pytest.mark.parametrize("name,K,N", synth.QWEN3_MOE_SHAPES)
def test_grouped_qwen3_moe_shapes(ops, B, name, K, N):
    """128 experts of the real shape, seeded top-8 routing of B tokens; the
    weights are drawn on the device and the checked experts' bf16 bits copied
    back for the oracle.  B = 1 .. 5 cross the launch rules of the small tiles
    (two column tiles per workgroup for one or two tokens, two waves per
    workgroup once the grid covers the CUs)."""
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


@pytest.mark.parametrize("T", [64, 512])
def test_grouped_overlapping_offsets_drop_items(ops, T):
    """Offsets that go back to 0: experts 0, 2, 4 and 6 each own all T rows, so
    the call has four times the items of a well-formed one and the items past
    the grid's bound min(E, T) + ceil(T / R) are dropped (16-row items at
    T = 64, the large tile at 512).  The call completes inside the output."""
    announce(f"qgemm_w4a16_grouped overlapping offsets T={T}")
    K, N, E = 256, 256, 8
    w_list = [synth.weights(K, N, seed=500 + e) for e in range(E)]
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(x) for x in w_list]))
    a = dev_bf16(synth.activations(T, K, seed=8))
    y = torch.full((T + 8, N), 7.0, dtype=torch.bfloat16, device="cuda")
    bad = torch.tensor([0, T, 0, T, 0, T, 0, T, T], dtype=torch.int32, device="cuda")
    gw(a, bad, out=y[:T])
    torch.cuda.synchronize()
    assert torch.all(y[T:] == 7.0)
    assert torch.all(torch.isfinite(y[:T].float()))
