"""The cross-workgroup K split of the W4A16 and 8-bit GEMMs, on a shared workspace.

Shapes whose tiles cannot fill the GPU split K across workgroups: each writes
its partial sums to a slot of the workspace and counts its arrival, and the
last arriver adds the slots.  These tests make every ordering or layout mistake
visible:

* before every call the slot region (everything after the 64 KiB counter
  region) is filled with NaN, so a slot read before its write lands in the
  output as a non-finite value;
* consecutive calls alternate between different activations, so a stale slot
  from the previous call would give the other input's answer;
* one workspace serves calls of different shapes in a row (M = 384, 512, 200
  at K = 14336, N = 4096), so counters must sit where no shape's slots reach.

Every output is checked for finiteness and against the CPU oracle (sampled
rows for the large shapes); the counters read zero after each call.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
from oracle import fp8_e4m3 as f8
from oracle import int4_g128 as q4
from oracle import int8 as i8
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 64 * 1024


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _poison_slots(ws, nbytes):
    """NaN over the workspace after the counter region (offset terms and slots)."""
    ws[COUNTER_BYTES:nbytes].view(torch.float32).fill_(float("nan"))


def _counters_zero(ws):
    return int(torch.count_nonzero(ws[:COUNTER_BYTES])) == 0


def _rows(M, n=40, seed=0):
    return np.unique(np.random.default_rng(seed + M).integers(0, M, n)) if M > n else np.arange(M)


def _split_of(name):
    return int(name.rsplit("S=", 1)[1])


# ------------------------------------------------------------------ W4A16

# decode K split (down at B = 9 / 16), large-M K split with 64-row tiles
# (M = 48, 200) and 128-row tiles (M = 384 at K = 28672)
W4A16_SPLIT = [(9, 14336, 4096), (16, 14336, 4096), (48, 14336, 4096), (200, 14336, 4096),
               (384, 28672, 8192)]


@pytest.mark.parametrize("M,K,N", W4A16_SPLIT)
def test_w4a16_split_alternating_inputs_nan_slots(ops, M, K, N):
    announce(f"qgemm_w4a16 split handoff, alternating inputs, NaN slots M={M} K={K} N={N}")
    name = ops.w4a16_kernel_for(M, N, K)
    assert _split_of(name) > 1, name
    w = synth.weights(K, N, seed=301 + K)
    codes, s = q4.quantize(w)
    lin = ops.W4A16Linear(ops.Int4G128Weight.from_bf16(dev_bf16(w)))
    ws, nbytes = lin.workspace(M)
    acts = [synth.activations(M, K, seed=311 + i) for i in range(2)]
    rows = _rows(M)
    refs = [q4.gemm_ref(a[rows], codes, s) for a in acts]
    first = [None, None]
    for rep in range(3):
        for i, a in enumerate(acts):
            _poison_slots(ws, nbytes)
            y = lin(dev_bf16(a))
            torch.cuda.synchronize()
            assert bool(torch.isfinite(y).all()), f"{name}: non-finite output (a slot read before its write)"
            assert _counters_zero(ws)
            yb = host_bits16(y)
            assert_close_rms(yb[rows], refs[i], what=f"{name} M={M} input {i} rep {rep}")
            if first[i] is None:
                first[i] = yb
            assert np.array_equal(yb, first[i])


def test_w4a16_one_workspace_across_shapes(ops):
    """M = 384, 512, 200 (K = 14336, N = 4096) on one W4A16Linear: the workspace
    grows to the largest need and is reused; 200 splits K over 64-row tiles."""
    K, N = 14336, 4096
    announce(f"qgemm_w4a16 one workspace across M = 384, 512, 200, 16, 384 (K={K} N={N})")
    w = synth.weights(K, N, seed=synth.weight_seed(0, 3))
    codes, s = q4.quantize(w)
    lin = ops.W4A16Linear(ops.Int4G128Weight.from_bf16(dev_bf16(w)))
    need = max(ops.w4a16_workspace_bytes(M, N, K) for M in (384, 512, 200, 16))
    lin._ws = torch.zeros(need, dtype=torch.uint8, device="cuda")    # one buffer for every shape
    a_all = synth.activations(512, K, seed=synth.activation_seed(0, 3))
    for M in (384, 512, 200, 16, 384):
        a = a_all[:M]
        y = lin(dev_bf16(a))
        torch.cuda.synchronize()
        assert lin._ws.numel() == need
        assert bool(torch.isfinite(y).all())
        assert _counters_zero(lin._ws)
        rows = _rows(M, seed=M)
        assert_close_rms(host_bits16(y)[rows], q4.gemm_ref(a[rows], codes, s),
                         what=f"{ops.w4a16_kernel_for(M, N, K)} M={M}")


# ------------------------------------------------------------------ 8-bit

# (M, K, N): 64 x 128 tiles with K split 2 / 8 / 5 ways (N = 1040 leaves a
# ragged last column tile) and 128 x 128 tiles split 4 ways
EIGHT_BIT_SPLIT = [(200, 14336, 4096), (100, 14336, 1040), (100, 10240, 1040), (300, 14336, 4096)]


def _eight_bit(ops, fmt):
    if fmt == "fp8":
        return (ops.W8A8Fp8Linear, ops.Fp8Weight, f8, ops.w8a8_workspace_bytes)
    return (ops.W8A8Int8Linear, ops.Int8Weight, i8, ops.w8a8_int8_workspace_bytes)


def _gemm_on_codes(ops, fmt, lin, a_dev):
    """The GEMM entry point on codes from the separate quantization kernel."""
    qa, sa = (ops.quantize_activations if fmt == "fp8" else ops.quantize_activations_int8)(a_dev)
    return lin(a_dev, qa=qa, sa=sa)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("M,K,N", EIGHT_BIT_SPLIT)
def test_8bit_split_alternating_inputs_nan_slots(ops, fmt, M, K, N):
    announce(f"qgemm_w8a8_{fmt} split handoff, alternating inputs, NaN slots M={M} K={K} N={N}")
    Lin, Weight, orc, ws_bytes = _eight_bit(ops, fmt)
    name = ops.w8a8_kernel_for(M, N, K)
    assert _split_of(name) > 1, name
    w = synth.weights(K, N, seed=401 + K + N)
    qw, sw = orc.quant_weight_per_channel(w)
    lin = Lin(Weight.from_bf16(dev_bf16(w)))
    ws, nbytes = lin.workspace(M)
    assert nbytes == ws_bytes(M, N, K) > COUNTER_BYTES
    acts = [synth.activations(M, K, seed=411 + i) for i in range(2)]
    rows = _rows(M)
    refs = []
    for a in acts:
        qa, sa = orc.quant_act_per_token(a[rows])
        refs.append(orc.gemm_ref(qa, sa, qw, sw))
    first = [None, None]
    for rep in range(3):
        for i, a in enumerate(acts):
            _poison_slots(ws, nbytes)
            y = _gemm_on_codes(ops, fmt, lin, dev_bf16(a))
            torch.cuda.synchronize()
            assert bool(torch.isfinite(y).all()), f"{name}: non-finite output (a slot read before its write)"
            assert _counters_zero(ws)
            yb = host_bits16(y)
            assert_close_rms(yb[rows], refs[i], what=f"{fmt} {name} M={M} input {i} rep {rep}")
            if first[i] is None:
                first[i] = yb
            assert np.array_equal(yb, first[i])


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_8bit_one_workspace_across_shapes(ops, fmt):
    K, N = 14336, 4096
    announce(f"qgemm_w8a8_{fmt} one workspace across M = 384, 512, 200, 384 (K={K} N={N})")
    Lin, Weight, orc, ws_bytes = _eight_bit(ops, fmt)
    w = synth.weights(K, N, seed=synth.weight_seed(0, 3))
    qw, sw = orc.quant_weight_per_channel(w)
    lin = Lin(Weight.from_bf16(dev_bf16(w)))
    need = max(ws_bytes(M, N, K) for M in (384, 512, 200))
    assert need > 0
    lin._ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    a_all = synth.activations(512, K, seed=synth.activation_seed(0, 3))
    for M in (384, 512, 200, 384):
        a = a_all[:M]
        y = _gemm_on_codes(ops, fmt, lin, dev_bf16(a))
        torch.cuda.synchronize()
        assert lin._ws.numel() == need
        assert bool(torch.isfinite(y).all())
        assert _counters_zero(lin._ws)
        rows = _rows(M, seed=M)
        qa, sa = orc.quant_act_per_token(a[rows])
        assert_close_rms(host_bits16(y)[rows], orc.gemm_ref(qa, sa, qw, sw),
                         what=f"{fmt} {ops.w8a8_kernel_for(M, N, K)} M={M}")
