"""W4A8-FP8 (INT4 g128 weights x dynamic per-token e4m3 activations): the
oracle (test infrastructure only).

What the pages fix ("When quantization pays", the mixture-of-experts section
and the engine configurations it quotes): mixed schemes put INT4 weights with
FP8 activations on the expert layers, which stay weight-stream bound at
serving batch.  The pages name the scheme and give no formulas, so this
oracle composes the two formats the other pages define:

W1  Weights: the INT4 g128 format of oracle.int4_g128 (abs-max scale per group
    of 128 input rows, bf16 scale, stored code = q + 8), unchanged.
W2  Activations: the dynamic per-token e4m3 quantization of oracle.fp8_e4m3
    (s_a = float32(amax) / 448, codes = e4m3(a / s_a)), unchanged.
W3  Output: Y = s_a[m] * sum_k dec(qa[m, k]) * w_hat[k, n] with w_hat the exact
    fp32 dequantized weight (code - 8) * s_g, formed in fp64.
"""
import numpy as np

from . import fp8_e4m3 as f8
from . import int4_g128 as q4


def gemm_ref(qa, sa, codes, scale_bits):
    """Y64 [M, N] = s_a[m] * dec(qa) @ w_hat (W3)."""
    a = f8.e4m3_decode(qa)
    w = q4.dequant_f32(codes, scale_bits).astype(np.float64)
    return (a @ w) * np.asarray(sa, np.float64)[:, None]


def grouped_gemm_ref(qa, sa, offsets, experts):
    """Per expert e (rows offsets[e] .. offsets[e+1]-1): gemm_ref on its rows.
    experts: {e: (codes, scale_bits)}.  Returns {e: Y64 [rows_e, N]}."""
    out = {}
    for e, (codes, s) in experts.items():
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        out[e] = gemm_ref(qa[r0:r1], sa[r0:r1], codes, s)
    return out


def gemm_bruteforce(qa, sa, codes, scale_bits):
    """Plain loops over python floats, for tiny shapes only."""
    table = f8.e4m3_decode_table()
    s = (np.asarray(scale_bits, np.uint32) << 16).view(np.float32)
    M, K = qa.shape
    N = codes.shape[1]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(table[qa[m, k]]) * ((int(codes[k, n]) - 8) * float(s[k // 128, n]))
            y[m, n] = acc * float(sa[m])
    return y
