"""qgemm_w8a8_fp8_dynamic / qgemm_w8a8_int8_dynamic: bf16 activations in, the
per-token quantization inside the call.

Their output equals the two-call path (quant_act_per_token (_int8), then
qgemm_w8a8_fp8 (_int8) on its codes) bit for bit, whether the small-M GEMM
quantizes the rows itself (up to 16 rows) or the codes go through the
workspace.  The activations carry rows that reach every branch of the fused
quantization: an all-zero row (scale 0, codes 0), a row of values near 1e30,
a row whose scale falls below 2^-100 (the code quotient by division), a row of
subnormal values (subnormal scale), and a row of exact code ties (scale 1).
Sampled rows of small shapes are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
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


def _fmt(ops, fmt):
    if fmt == "fp8":
        return ops.Fp8Weight, ops.W8A8Fp8Linear, ops.quantize_activations, f8, 448.0
    return ops.Int8Weight, ops.W8A8Int8Linear, ops.quantize_activations_int8, i8, 127.0


def _activations(M, K, qmax, seed):
    """N(0, 1) rows, then the special rows in order while there is room."""
    x = synth.normal_bf16((M, K), seed).view(np.uint16)
    f = (x.astype(np.uint32) << 16).view(np.float32).copy()
    rng = np.random.default_rng(seed)
    special = [
        np.zeros(K, np.float32),                                        # scale 0
        rng.standard_normal(K).astype(np.float32) * np.float32(1e30),    # large scale (fp32 epilogue stays finite)
        rng.standard_normal(K).astype(np.float32) * np.float32(1e-33),   # scale < 2^-100
        rng.standard_normal(K).astype(np.float32) * np.float32(1e-39),   # subnormal values and scale
    ]
    ties = np.resize(np.array([qmax, 1.0625, 1.1875, -2.125, 0.5, 1.5, -2.5, 3.0], np.float32), K)
    special.append(ties)                                                # scale exactly 1: code ties
    for j, row in enumerate(special[: max(0, M - 1)]):
        f[1 + j] = row
    return f32_to_bf16_bits(f)


_W = {}


def _weight(ops, fmt, K, N):
    key = (fmt, K, N)
    if key not in _W:
        if len(_W) > 6:
            _W.clear()
        Weight = _fmt(ops, fmt)[0]
        small = K * N <= (1 << 22)
        w_bits = synth.weights(K, N, seed=911 + K + N) if small else None
        w_dev = dev_bf16(w_bits) if small else synth.normal_bf16_device((K, N), 911 + K + N,
                                                                          synth.WEIGHT_STD, "cuda")
        _W[key] = (Weight.from_bf16(w_dev), w_bits)
    return _W[key]


def _both(ops, fmt, M, K, N, seed):
    _, Lin, quant, _, qmax = _fmt(ops, fmt)
    wt, w_bits = _weight(ops, fmt, K, N)
    a_bits = _activations(M, K, qmax, seed)
    a = dev_bf16(a_bits)
    lin = Lin(wt)
    qa, sa = quant(a)
    y_two = host_bits16(lin(a, qa=qa, sa=sa))
    y_dyn = host_bits16(lin(a))
    torch.cuda.synchronize()
    return y_two, y_dyn, a_bits, w_bits


# (K, N): one and two column tiles per workgroup, long K, K below 512-multiples (never fused)
SHAPES = [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096), (1024, 272), (1536, 2048), (384, 1040)]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("K,N", SHAPES)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 6, 8, 16, 17, 40])
def test_dynamic_equals_two_calls(ops, fmt, M, K, N):
    kern = ops.w8a8_dynamic_kernel_for(M, N, K)
    announce(f"qgemm_w8a8_{fmt}_dynamic M={M} K={K} N={N} ({kern})")
    y_two, y_dyn, _, _ = _both(ops, fmt, M, K, N, seed=17 + M + K)
    assert np.array_equal(y_dyn, y_two), f"{fmt} M={M} K={K} N={N} {kern}"


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("M,K,N", [(1, 1024, 272), (6, 1536, 2048), (16, 1024, 272), (3, 384, 1040)])
def test_dynamic_against_oracle(ops, fmt, M, K, N):
    """Special rows included: zero, huge, tiny, subnormal and tie rows."""
    announce(f"qgemm_w8a8_{fmt}_dynamic vs oracle M={M} K={K} N={N}")
    orc = _fmt(ops, fmt)[3]
    _, y_dyn, a_bits, w_bits = _both(ops, fmt, M, K, N, seed=29 + M)
    qa, sa = orc.quant_act_per_token(a_bits)
    qw, sw = orc.quant_weight_per_channel(w_bits)
    ref = orc.gemm_ref(qa, sa, qw, sw)
    # each row against its own output RMS (their scales span 1e-35 .. 1e35); the
    # zero row must give zeros; the subnormal row's outputs lie below bf16's
    # normal range, where the output rounding alone exceeds the tolerance, so
    # it is covered by the bit-exact comparison with the two-call path only
    for m in range(M):
        peak = float(np.max(np.abs(ref[m])))
        if peak == 0.0:
            np.testing.assert_array_equal(y_dyn[m] & 0x7fff, 0)
        elif peak > 1e-30:
            assert_close_rms(y_dyn[m:m + 1], ref[m:m + 1], what=f"{fmt} dynamic row {m}")


def test_fused_where_expected(ops):
    """The 8B decode shapes that quantize inside the GEMM: all of them at one
    row, qkv and o (one round of workgroups) up to four rows, gate_up (two
    rounds) up to three, long-K down at one row only (registers)."""
    fused = lambda M, K, N: ops.w8a8_dynamic_kernel_for(M, N, K).startswith("w8a8_small_m_dyn_kernel<")
    for K, N in [(4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096), (4096, 128256)]:
        assert fused(1, K, N), (K, N)
    assert fused(4, 4096, 6144) and fused(4, 4096, 4096) and not fused(5, 4096, 4096)
    assert fused(3, 4096, 28672) and not fused(4, 4096, 28672)
    assert not fused(2, 14336, 4096) and not fused(16, 4096, 4096)
    assert not fused(17, 4096, 4096) and not fused(1, 384, 1040)
    assert ops.w8a8_dynamic_workspace_bytes(1, 4096, 4096) == 0
    assert ops.w8a8_dynamic_workspace_bytes(16, 4096, 4096) >= 16 * 4096


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_dynamic_deterministic_and_workspace_reuse(ops, fmt):
    """One linear serves fused and unfused row counts in turn on one workspace."""
    announce(f"qgemm_w8a8_{fmt}_dynamic workspace reuse")
    _, Lin, quant, _, qmax = _fmt(ops, fmt)
    wt, _ = _weight(ops, fmt, 4096, 4096)
    lin = Lin(wt)
    for M in (40, 1, 16, 300, 4, 40):
        a = dev_bf16(_activations(M, 4096, qmax, seed=M))
        qa, sa = quant(a)
        y_two = host_bits16(lin(a, qa=qa, sa=sa))
        y1 = host_bits16(lin(a))
        y2 = host_bits16(lin(a))
        assert np.array_equal(y1, y_two) and np.array_equal(y2, y_two), (fmt, M)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_unfused_codes_leave_the_counters_alone(ops, fmt):
    """One workspace, a bench step's order: 16 rows (unfused: codes in the
    workspace, the GEMM itself needs none), then 200 rows at K = 14336 whose
    GEMM splits K and counts arrivals in the counter region.  The codes must
    never land in that region: it reads zero after the 16-row call, and the
    split call matches the two-call path on a fresh workspace."""
    announce(f"qgemm_w8a8_{fmt}_dynamic counter region after an unfused call")
    _, Lin, quant, _, qmax = _fmt(ops, fmt)
    K, N = 14336, 4096
    wt, _ = _weight(ops, fmt, K, N)
    lin = Lin(wt)
    need = max(ops.w8a8_dynamic_workspace_bytes(M, N, K) for M in (16, 200))
    lin._ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    assert "S=" in ops.w8a8_kernel_for(200, N, K) and not ops.w8a8_kernel_for(200, N, K).endswith("S=1")
    for M in (16, 200, 16, 200):
        a = dev_bf16(_activations(M, K, qmax, seed=500 + M))
        y = host_bits16(lin(a))
        torch.cuda.synchronize()
        assert lin._ws.numel() == need
        assert int(torch.count_nonzero(lin._ws[:65536])) == 0, f"counter region written (M={M})"
        ref_lin = Lin(wt)
        qa, sa = quant(a)
        assert np.array_equal(y, host_bits16(ref_lin(a, qa=qa, sa=sa))), (fmt, M)

