"""Pins of the expert-grouped W4A16 oracle and of the routing generator.

Pins: brute force on a tiny ragged grouping with empty experts, the special
case of one expert owning every row (the plain product), identical experts
(the plain product over the whole batch), and the routing invariants (k
distinct experts per token, offsets that partition the rows, the expected
B k / E rows per expert on average)."""
import numpy as np

from oracle import int4_g128 as q4
from weight_only_quantized_w4a16_amd import synth


def _experts(E, K, N, seed):
    return {e: q4.quantize(synth.weights(K, N, seed=seed + e)) for e in range(E)}


def test_bruteforce_tiny_ragged():
    E, K, N = 5, 256, 16
    offsets = np.array([0, 3, 3, 4, 9, 9], dtype=np.int32)          # experts 1 and 4 empty
    a = synth.activations(9, K, seed=1)
    ex = _experts(E, K, N, seed=10)
    y = q4.grouped_gemm_ref(a, offsets, ex)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        assert y[e].shape == (r1 - r0, N)
        if r1 > r0:
            ref = q4.gemm_bruteforce(a[r0:r1], *ex[e])
            assert np.allclose(y[e], ref, rtol=1e-12, atol=1e-12)


def test_one_expert_owns_all_rows():
    K, N, T = 512, 48, 7
    a = synth.activations(T, K, seed=2)
    ex = _experts(3, K, N, seed=20)
    offsets = np.array([0, 0, T, T], dtype=np.int32)
    y = q4.grouped_gemm_ref(a, offsets, ex)
    assert np.array_equal(y[1], q4.gemm_ref(a, *ex[1]))
    assert y[0].shape == (0, N) and y[2].shape == (0, N)


def test_identical_experts_equal_the_plain_product():
    K, N, T = 384, 32, 12
    a = synth.activations(T, K, seed=3)
    one = q4.quantize(synth.weights(K, N, seed=30))
    offsets = np.array([0, 2, 2, 7, 12], dtype=np.int32)
    y = q4.grouped_gemm_ref(a, offsets, {e: one for e in range(4)})
    stacked = np.concatenate([y[e] for e in range(4)], axis=0)
    assert np.allclose(stacked, q4.gemm_ref(a, *one), rtol=0, atol=1e-12)


def test_routing_invariants():
    B, E, k = 256, 128, 8
    token, offsets = synth.moe_routing(B, E, k, seed=4)
    assert offsets[0] == 0 and offsets[-1] == B * k and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.bincount(token, minlength=B), np.full(B, k))
    for e in range(E):
        t = token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(t) > 0)                    # each token at most once per expert
    seen = np.zeros((B, E), dtype=int)
    for e in range(E):
        seen[token[offsets[e]:offsets[e + 1]], e] += 1
    assert np.all(seen.sum(axis=1) == k) and seen.max() == 1
    assert abs(np.diff(offsets).mean() - B * k / E) < 1e-9
