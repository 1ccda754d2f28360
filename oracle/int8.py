"""W8A8-INT8: the oracle (test infrastructure only).

What the pages fix ("Give Me BF16 or Give Me Death", section 3.4,
"W8A8-INT Quantization" and the activation-quantization paragraphs)
--------------------------------------------------------------------
* Weights: symmetric, one scale per output channel, no zero point,
  w_hat = s * round(w / s) with s = max|w| / 127; codes span [-127, 127]
  (-128 is left unused by the symmetric scheme).
* Activations (8B and 405B models): dynamic per-token quantization, each token
  row with its own scale from its own range, the same symmetric 8-bit map.
* The product runs on 8-bit integers with a higher-precision (32-bit integer)
  accumulator and is dequantized back to 16 bits.

Readings where the pages are silent (listed with the design notes)
------------------------------------------------------------------
I1  Scales are fp32: s = float32(amax) / 127 (IEEE division).  The element is
    divided by s in fp32 and the quotient rounded half to even, then clamped
    to [-127, 127] (the quotient exceeds 127 by at most a rounding step).
I2  A row or column whose amax is 0 stores scale 0 and codes 0.
I3  Output channel = column n of W [K, N]; activations [M, K], one scale per row.
I4  Output: Y = s_a[m] * s_w[n] * sum_k qa[m, k] qw[k, n]; the integer sum is
    exact (|sum| <= 127^2 K fits 32 bits for K <= 131072), the oracle forms
    the product in fp64.
I5  Native weight order: the fp8 path's order (module oracle.fp8_e4m3), byte
    for byte, with int8 codes in place of e4m3 codes.

GPTQ's error compensation and SmoothQuant need calibration activations and are
not part of this oracle: the weights are quantized round-to-nearest.
"""
import numpy as np

from .bf16 import bf16_bits_to_f32

QMAX = 127.0
MAX_K = 131072


def _quantize(x, axis):
    """Symmetric int8 along `axis` (I1, I2): returns (codes int8, s fp32)."""
    amax = np.max(np.abs(x), axis=axis)
    s = (amax.astype(np.float32) / np.float32(QMAX)).astype(np.float32)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    shape = [1, 1]
    shape[1 - axis] = -1
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.rint((x / s_safe.reshape(shape)).astype(np.float32))
    q = np.clip(q, -QMAX, QMAX)
    q = np.where(zero.reshape(shape), 0.0, q)
    return q.astype(np.int8), s


def quant_act_per_token(a_bits):
    """bf16 activations [M, K] -> (codes int8 [M, K], s fp32 [M])."""
    return _quantize(bf16_bits_to_f32(a_bits), axis=1)


def quant_weight_per_channel(w_bits):
    """bf16 weights [K, N] -> (codes int8 [K, N], s fp32 [N])."""
    return _quantize(bf16_bits_to_f32(w_bits), axis=0)


def gemm_ref(qa, sa, qw, sw):
    """Y64[m, n] = s_a[m] * s_w[n] * sum_k qa[m, k] qw[k, n] (I4): exact integer sum.

    The sum is formed by an fp64 matrix product, which is exact here: every
    product and every partial sum is an integer of magnitude at most
    127^2 * K < 2^31, far inside fp64's 2^53 exact-integer range.
    """
    if qa.shape[1] > MAX_K:
        raise ValueError(f"K={qa.shape[1]} exceeds the int32 accumulator bound {MAX_K}")
    acc = np.asarray(qa, np.float64) @ np.asarray(qw, np.float64)
    return acc * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def gemm_bruteforce(qa, sa, qw, sw):
    """Plain loops over python ints, for tiny shapes only."""
    M, K = qa.shape
    N = qw.shape[1]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0
            for k in range(K):
                acc += int(qa[m, k]) * int(qw[k, n])
            y[m, n] = acc * float(sa[m]) * float(sw[n])
    return y
