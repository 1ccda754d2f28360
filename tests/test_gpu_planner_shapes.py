"""Shapes whose launch plans the model shapes never reach: K with an odd or
prime number of 128-row groups (7, 45 = 3^2 * 5, 144 = 2^4 * 3^2), so that
K splits take the divisors those counts allow (the decode kernel split 5, 6
or 9 ways, the large-M kernel 3, 4, 5 or 8 ways) or none at all, at row
counts from decode (1, 9, 16) through the small-M kernel (40) to large M
(100, 300).

W4A16, W8A8-FP8 and W8A8-INT8 (bf16 activations in, quantized inside the
call or by the separate kernel) against the CPU oracle on sampled rows over
all N columns: max |err| <= 2e-2 x RMS of the fp64 oracle rows.
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

N = 4096
KS = [896, 5760, 18432]
MS = [1, 9, 16, 40, 100, 300]


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


_CACHE = {}


def _weights(K):
    """bf16 weight bits of [K, N] and the activations for the largest M."""
    if K not in _CACHE:
        _CACHE[K] = (synth.weights(K, N, seed=900 + K), synth.activations(max(MS), K, seed=901 + K))
    return _CACHE[K]


def _rows(M):
    return np.unique(np.concatenate([np.random.default_rng(M).integers(0, M, 12), [M - 1]]))


@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("M", MS)
def test_w4a16_planner_shapes(ops, M, K):
    kern = ops.w4a16_kernel_for(M, N, K)
    announce(f"qgemm_w4a16 M={M} K={K} (G={K // 128}) N={N} ({kern})")
    w, a_all = _weights(K)
    key = ("w4", K)
    if key not in _CACHE:
        _CACHE[key] = (ops.Int4G128Weight.from_bf16(dev_bf16(w)), q4.quantize(w))
    wt, (codes, s) = _CACHE[key]
    a = a_all[:M]
    y = host_bits16(ops.W4A16Linear(wt)(dev_bf16(a)))
    rows = _rows(M)
    assert_close_rms(y[rows], q4.gemm_ref(a[rows], codes, s), what=f"w4a16 M={M} K={K} {kern}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("K", KS)
@pytest.mark.parametrize("M", MS)
def test_w8a8_planner_shapes(ops, fmt, M, K):
    kern = ops.w8a8_dynamic_kernel_for(M, N, K)
    announce(f"qgemm_w8a8_{fmt}_dynamic M={M} K={K} (G={K // 128}) N={N} ({kern})")
    orc = f8 if fmt == "fp8" else i8
    Weight = ops.Fp8Weight if fmt == "fp8" else ops.Int8Weight
    Lin = ops.W8A8Fp8Linear if fmt == "fp8" else ops.W8A8Int8Linear
    w, a_all = _weights(K)
    key = (fmt, K)
    if key not in _CACHE:
        _CACHE[key] = (Weight.from_bf16(dev_bf16(w)), orc.quant_weight_per_channel(w))
    wt, (qw, sw) = _CACHE[key]
    a = a_all[:M]
    y = host_bits16(Lin(wt)(dev_bf16(a)))
    rows = _rows(M)
    qa, sa = orc.quant_act_per_token(a[rows])
    assert_close_rms(y[rows], orc.gemm_ref(qa, sa, qw, sw), what=f"{fmt} M={M} K={K} {kern}")
