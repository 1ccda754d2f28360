"""Seeded random shapes across the launch planners: every GEMM entry point picks
its kernel, tile shape, K split and grid from (M, N, K) (and, grouped, from the
routing), so shapes drawn at random reach combinations that the model shapes
do not.  Each case compares sampled output rows over all N columns with the
CPU oracle: max |err| <= 2e-2 x RMS of the fp64 oracle rows.

Shapes: M in 1 .. 1100, N a multiple of 16 up to 3072, K a multiple of 128 up
to 6144; grouped calls with 1 .. 40 experts, 1 .. 1200 routed rows and routing
that leaves some experts empty (so both the small and the large grouped tiles
run).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
from oracle import fp8_e4m3 as f8
from oracle import int4_g128 as q4
from oracle import int8 as i8
from oracle import w4a8
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu

N_DENSE = 40
N_GROUPED = 24


def _dense_shapes(seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(N_DENSE):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 401)),
                            int(rng.integers(401, 1101))]))
        N = 16 * int(rng.integers(1, 193))
        K = 128 * int(rng.integers(1, 49))
        out.append((M, N, K))
    return out


def _grouped_cases(seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(N_GROUPED):
        E = int(rng.integers(1, 41))
        T = int(rng.integers(1, 1201))
        # routing: T rows over E experts, a random share of the experts empty
        active = rng.random(E) < 0.7
        if not active.any():
            active[int(rng.integers(0, E))] = True
        w = rng.random(E) * active
        sizes = rng.multinomial(T, w / w.sum())
        N = 16 * int(rng.integers(1, 97))
        K = 128 * int(rng.integers(1, 17))
        out.append((E, T, [int(x) for x in sizes], N, K))
    return out


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


def _rows(M, seed):
    return np.unique(np.concatenate([np.random.default_rng(seed).integers(0, M, 6), [0, M - 1]]))


@pytest.mark.parametrize("i,shape", list(enumerate(_dense_shapes(2024))))
def test_w4a16_random_shape(ops, i, shape):
    M, N, K = shape
    kern = ops.w4a16_kernel_for(M, N, K)
    announce(f"qgemm_w4a16 random #{i} M={M} N={N} K={K} ({kern})")
    w = synth.weights(K, N, seed=3000 + i)
    a = synth.activations(M, K, seed=4000 + i)
    wt = ops.Int4G128Weight.from_bf16(dev_bf16(w))
    y = host_bits16(ops.W4A16Linear(wt)(dev_bf16(a)))
    codes, s = q4.quantize(w)
    rows = _rows(M, i)
    assert_close_rms(y[rows], q4.gemm_ref(a[rows], codes, s), what=f"w4a16 M={M} N={N} K={K} {kern}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("i,shape", list(enumerate(_dense_shapes(2025)))[:20])
def test_w8a8_dynamic_random_shape(ops, fmt, i, shape):
    M, N, K = shape
    kern = ops.w8a8_dynamic_kernel_for(M, N, K)
    announce(f"qgemm_w8a8_{fmt}_dynamic random #{i} M={M} N={N} K={K} ({kern})")
    orc = f8 if fmt == "fp8" else i8
    Weight = ops.Fp8Weight if fmt == "fp8" else ops.Int8Weight
    Lin = ops.W8A8Fp8Linear if fmt == "fp8" else ops.W8A8Int8Linear
    w = synth.weights(K, N, seed=5000 + i)
    a = synth.activations(M, K, seed=6000 + i)
    y = host_bits16(Lin(Weight.from_bf16(dev_bf16(w)))(dev_bf16(a)))
    qw, sw = orc.quant_weight_per_channel(w)
    rows = _rows(M, i)
    qa, sa = orc.quant_act_per_token(a[rows])
    assert_close_rms(y[rows], orc.gemm_ref(qa, sa, qw, sw), what=f"{fmt} M={M} N={N} K={K} {kern}")


@pytest.mark.parametrize("i,case", list(enumerate(_grouped_cases(2026))))
def test_grouped_random_routing(ops, i, case):
    E, T, sizes, N, K = case
    announce(f"qgemm_w4a16_grouped random #{i} E={E} T={T} N={N} K={K} sizes={sizes}")
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    a = synth.activations(T, K, seed=7000 + i)
    w = synth.normal_bf16_device((E, K, N), seed=8000 + i, std=synth.WEIGHT_STD, device="cuda")
    gw = ops.GroupedInt4Weight.from_bf16(w)
    off = torch.from_numpy(offsets).cuda()
    y = host_bits16(gw(dev_bf16(a), off))
    nonempty = [e for e in range(E) if sizes[e] > 0]
    for e in nonempty[:: max(1, len(nonempty) // 4)]:
        r0, r1 = offsets[e], offsets[e + 1]
        ref = q4.grouped_gemm_ref(a, offsets, {e: q4.quantize(host_bits16(w[e]))})[e]
        assert_close_rms(y[r0:r1], ref, what=f"grouped E={E} T={T} N={N} K={K} expert {e}")
    # W4A8 on the same routing (bf16 rows in, per-token e4m3 inside the call)
    y8 = host_bits16(gw.w4a8_dynamic(dev_bf16(a), off))
    for e in nonempty[:: max(1, len(nonempty) // 4)]:
        r0, r1 = offsets[e], offsets[e + 1]
        qa, sa = f8.quant_act_per_token(a[r0:r1])
        ref = w4a8.gemm_ref(qa, sa, *q4.quantize(host_bits16(w[e])))
        assert_close_rms(y8[r0:r1], ref, what=f"w4a8 grouped E={E} T={T} N={N} K={K} expert {e}")
