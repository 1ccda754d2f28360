"""qgemm_w4a16_noalloc (the allocation-free variant, whose workspace is the
library's own per-device scratch array) against qgemm_w4a16 with a caller
workspace, through the C ABI.

Both entry points run the same kernels with the same plans, so their outputs
must agree bit for bit; each output is also checked against the CPU oracle on
sampled rows (max |err| <= 2e-2 x RMS).  Every case makes two calls in a row,
the second with fewer rows, so the second call runs on the scratch contents
the first one left.  A shape whose workspace exceeds the scratch is rejected
before any launch.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import announce, assert_close_rms, dev_bf16, host_bits16
from oracle import int4_g128 as q4
from weight_only_quantized_w4a16_amd import synth

pytestmark = pytest.mark.gpu

QG_ERR_WORKSPACE = 4


@pytest.fixture(scope="module")
def ops():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from weight_only_quantized_w4a16_amd import ops as _ops
    return _ops


# (K, N, first M, second M): the decode K split, the large-M K split over
# 64-row tiles, large-M tiles without a split (offset terms only), and a
# shape that needs no workspace at all
CASES = [(14336, 4096, 16, 9), (14336, 4096, 200, 100), (4096, 4096, 1024, 512), (4096, 6144, 4, 1)]


@pytest.mark.parametrize("K,N,M1,M2", CASES)
def test_noalloc_matches_workspace_entry_point(ops, K, N, M1, M2):
    w = synth.weights(K, N, seed=501 + K + N)
    codes, s = q4.quantize(w)
    wt = ops.Int4G128Weight.from_bf16(dev_bf16(w))
    a_all = synth.activations(M1, K, seed=503 + M1)
    for M in (M1, M2):
        need = ops.w4a16_workspace_bytes(M, N, K)
        announce(f"qgemm_w4a16_noalloc M={M} K={K} N={N} ({ops.w4a16_kernel_for(M, N, K)}, "
                 f"workspace {need} bytes)")
        assert need <= ops.NOALLOC_SCRATCH_BYTES
        a = dev_bf16(a_all[:M])
        y_ref = ops.W4A16Linear(wt)(a)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        y.fill_(float("nan"))
        ops.qgemm_w4a16_noalloc(a, wt.packed, wt.scales, y, M, N, K)
        torch.cuda.synchronize()
        got, ref_bits = host_bits16(y), host_bits16(y_ref)
        assert np.array_equal(got, ref_bits), f"noalloc differs from qgemm_w4a16 at M={M}"
        rows = np.unique(np.random.default_rng(M).integers(0, M, 40))
        assert_close_rms(got[rows], q4.gemm_ref(a_all[rows], codes, s), what=f"noalloc M={M} K={K} N={N}")


def test_noalloc_rejects_a_workspace_beyond_the_scratch(ops):
    """M = 8192, K = 131072: the offset terms alone (1024 groups x 8192 rows x 4
    bytes) fill the 32 MiB scratch, so the call is refused before any launch.
    The buffers are allocated at their full sizes all the same."""
    M, K, N = 8192, 131072, 16
    need = ops.w4a16_workspace_bytes(M, N, K)
    announce(f"qgemm_w4a16_noalloc refuses M={M} K={K} N={N} (workspace {need} bytes)")
    assert need > ops.NOALLOC_SCRATCH_BYTES
    a = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    packed = torch.zeros(K * N // 8, dtype=torch.int32, device="cuda")
    scales = torch.zeros(K // 128 * N, dtype=torch.int16, device="cuda")
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.QGemmError) as e:
        ops.qgemm_w4a16_noalloc(a, packed, scales, y, M, N, K)
    assert e.value.status == QG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
