"""GPU parity of the W4A8-FP8 path (INT4 g128 weights x per-token e4m3
activations) against the oracle, dense and expert-grouped: max |err| <= 2e-2 x
RMS of the fp64 oracle output per call (per expert for the grouped form)."""
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


def _dense(ops, a_bits, w_bits):
    lin = ops.W4A8Linear(ops.Int4G128Weight.from_bf16(dev_bf16(w_bits)))
    y = lin(dev_bf16(a_bits))
    torch.cuda.synchronize()
    return host_bits16(y)


@pytest.mark.parametrize("K,N", [(128, 16), (256, 48), (1280, 144), (4096, 512)])
@pytest.mark.parametrize("M", [1, 5, 16, 17, 40, 64, 100])
def test_w4a8_parity(ops, M, K, N):
    announce(f"qgemm_w4a8_fp8 M={M} K={K} N={N}")
    w = synth.weights(K, N, seed=17 + K + N)
    a = synth.activations(M, K, seed=19 + M)
    qa, sa = f8.quant_act_per_token(a)
    codes, s = q4.quantize(w)
    y = _dense(ops, a, w)
    assert_close_rms(y, w4a8.gemm_ref(qa, sa, codes, s), what=f"w4a8 M={M} K={K} N={N}")


def test_w4a8_every_code_and_subnormal_activation(ops):
    """Weights that take all 15 abs-max codes (1..15; the codes 1..7 are e4m3
    subnormals on the MFMA), and activation rows that hold e4m3 subnormals."""
    announce("qgemm_w4a8_fp8 all codes, subnormal activations")
    K, N = 256, 32
    rng = np.random.default_rng(2)
    levels = np.arange(-7, 8, dtype=np.float32)
    w = levels[rng.integers(0, 15, (K, N))] * np.float32(0.01)
    w[0::128, :] = 0.07                              # abs-max 0.07: s = bf16(0.01), every level reachable
    wb = f32_to_bf16_bits(w)
    table = f8.e4m3_decode_table()
    a = rng.choice(table[1:16], size=(8, K)) * rng.choice([-1.0, 1.0], size=(8, K))
    a[:, 0] = 448.0                                  # s_a = 1: codes are the values themselves
    ab = f32_to_bf16_bits(a)
    qa, sa = f8.quant_act_per_token(ab)
    assert np.all(sa == 1.0)
    codes, s = q4.quantize(wb)
    assert len(np.unique(codes)) == 15
    y = _dense(ops, ab, wb)
    assert_close_rms(y, w4a8.gemm_ref(qa, sa, codes, s), what="w4a8 all codes")


@pytest.mark.parametrize("j,name,K,N", [(0, "qkv", 4096, 6144), (3, "down", 14336, 4096)])
@pytest.mark.parametrize("B", [1, 16, 64])
def test_w4a8_llama3_shapes_sampled(ops, B, j, name, K, N):
    announce(f"qgemm_w4a8_fp8 8B {name} B={B}")
    w = synth.weights(K, N, seed=synth.weight_seed(0, j))
    a = synth.activations(B, K, seed=synth.activation_seed(0, j))
    y = _dense(ops, a, w)
    cols = np.unique(np.random.default_rng(B).integers(0, N, 96))
    qa, sa = f8.quant_act_per_token(a)
    codes, s = q4.quantize(w[:, cols])
    assert_close_rms(y[:, cols], w4a8.gemm_ref(qa, sa, codes, s), what=f"w4a8 {name} B={B}")


# means of 17, 2 and 44 routed rows per expert (T / min(E, T)): 32- and 16-row
# items on the small tiles (N < 256), then, from a mean of 17 rows and
# N >= 256, 64-row items on the large tile (64 x 256, K through LDS stages):
# N = 272 leaves a last workgroup with one 16-column tile, K = 640 five groups
# (not a multiple of the three stages); items of 1, 7 and 33 rows leave the
# second row of waves without rows
@pytest.mark.parametrize("sizes,K,N", [([0, 1, 17, 0, 40, 3, 70, 5], 256, 64),
                                       ([2, 0, 0, 5, 1, 0, 3, 0, 0, 4], 384, 48),
                                       ([0, 65, 33, 0, 128, 7, 70], 384, 256),
                                       ([0, 65, 33, 0, 128, 7, 70], 640, 272)])
def test_w4a8_grouped_ragged(ops, sizes, K, N):
    announce(f"qgemm_w4a8_fp8_grouped sizes={sizes} K={K} N={N}")
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(offsets[-1])
    w_list = [synth.weights(K, N, seed=400 + e) for e in range(len(sizes))]
    a = synth.activations(T, K, seed=T + 3)
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(x) for x in w_list]))
    qa_d, sa_d = ops.quantize_activations(dev_bf16(a))
    y = host_bits16(gw.w4a8(qa_d, sa_d, torch.from_numpy(offsets).cuda()))
    qa, sa = f8.quant_act_per_token(a)
    for e in range(len(sizes)):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            ref = w4a8.grouped_gemm_ref(qa, sa, offsets, {e: q4.quantize(w_list[e])})[e]
            assert_close_rms(y[r0:r1], ref, what=f"w4a8 expert {e}")


@pytest.mark.parametrize("j", [0, 1])
@pytest.mark.parametrize("B", [1, 8, 16, 64, 1024])
def test_w4a8_grouped_qwen3_shapes(ops, B, j):
    E, k = synth.QWEN3_MOE_EXPERTS, synth.QWEN3_MOE_TOPK
    name, K, N = synth.QWEN3_MOE_SHAPES[j]
    announce(f"qgemm_w4a8_fp8_grouped qwen3 {name} B={B}")
    token, offsets = synth.moe_routing(B, E, k, seed=B)
    a = synth.activations(B, K, seed=11 + B)[token]
    w = synth.normal_bf16_device((E, K, N), seed=77 + j, std=synth.WEIGHT_STD, device="cuda")
    gw = ops.GroupedInt4Weight.from_bf16(w)
    qa_d, sa_d = ops.quantize_activations(dev_bf16(a))
    y = host_bits16(gw.w4a8(qa_d, sa_d, torch.from_numpy(offsets).cuda()))
    qa, sa = f8.quant_act_per_token(a)
    nonempty = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    for e in nonempty[:: max(1, len(nonempty) // 5)]:
        r0, r1 = offsets[e], offsets[e + 1]
        ref = w4a8.grouped_gemm_ref(qa, sa, offsets, {e: q4.quantize(host_bits16(w[e]))})[e]
        assert_close_rms(y[r0:r1], ref, what=f"w4a8 qwen3 B={B} expert {e}")


# several experts per lane of the work-item derivation (E = 1000 and 300):
# 16-row items, the quantization inside the call (fewer than 48 rows), and
# the large tile
@pytest.mark.parametrize("E,T,K,N", [(1000, 600, 128, 16), (1000, 40, 128, 16), (300, 12000, 128, 272)])
def test_w4a8_grouped_many_experts(ops, E, T, K, N):
    announce(f"qgemm_w4a8_fp8_grouped(_dynamic) many experts E={E} T={T} K={K} N={N}")
    rng = np.random.default_rng(E + T)
    p = rng.random(E) ** 3
    p[rng.random(E) < 0.3] = 0.0
    p[rng.integers(E)] += 1e-3
    sizes = rng.multinomial(T, p / p.sum())
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    w_list = [synth.weights(K, N, seed=2000 + e) for e in range(E)]
    a = synth.activations(T, K, seed=E + 1)
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(x) for x in w_list]))
    off = torch.from_numpy(offsets).cuda()
    qa_d, sa_d = ops.quantize_activations(dev_bf16(a))
    y = host_bits16(gw.w4a8(qa_d, sa_d, off))
    y_dyn = host_bits16(gw.w4a8_dynamic(dev_bf16(a), off))
    assert np.array_equal(y_dyn, y)
    qa, sa = f8.quant_act_per_token(a)
    nonempty = [e for e in range(E) if sizes[e] > 0]
    for e in nonempty[:: max(1, len(nonempty) // 8)] + [nonempty[-1]]:
        r0, r1 = offsets[e], offsets[e + 1]
        ref = w4a8.grouped_gemm_ref(qa, sa, offsets, {e: q4.quantize(w_list[e])})[e]
        assert_close_rms(y[r0:r1], ref, what=f"w4a8 E={E} expert {e}")


@pytest.mark.parametrize("T", [40, 64, 512])
def test_w4a8_grouped_overlapping_offsets_drop_items(ops, T):
    """Offsets that go back to 0 (experts 0, 2, 4 and 6 each own all T rows):
    four times the items of well-formed offsets, the items past the grid's
    bound dropped.  The two-call and the bf16-input entry points (quantization
    inside the GEMM at 40 rows, on the large tile at 512) complete inside the
    output."""
    announce(f"qgemm_w4a8_fp8_grouped(_dynamic) overlapping offsets T={T}")
    K, N, E = 256, 256, 8
    gw = ops.GroupedInt4Weight.from_bf16(torch.stack([dev_bf16(synth.weights(K, N, seed=700 + e))
                                                      for e in range(E)]))
    a = dev_bf16(synth.activations(T, K, seed=9))
    bad = torch.tensor([0, T, 0, T, 0, T, 0, T, T], dtype=torch.int32, device="cuda")
    qa, sa = ops.quantize_activations(a)
    for call in (lambda out: gw.w4a8(qa, sa, bad, out=out), lambda out: gw.w4a8_dynamic(a, bad, out=out)):
        y = torch.full((T + 8, N), 7.0, dtype=torch.bfloat16, device="cuda")
        call(y[:T])
        torch.cuda.synchronize()
        assert torch.all(y[T:] == 7.0)
        assert torch.all(torch.isfinite(y[:T].float()))
