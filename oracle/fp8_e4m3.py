"""W8A8-FP8: the oracle (test infrastructure only).

What the pages fix ("Give Me BF16 or Give Me Death", section 3.4,
"W8A8-FP Quantization")
----------------------------------------------------------------
* Weights: symmetric, one scale per output channel, no zero point,
  Q(x) = s * rnd(x / s) with s = max|x| / q_max and rnd to the nearest FP8
  value.
* Activations: dynamic per-token, the same formula applied to each token row
  with its own scale computed on the fly.
* The quantized operands go straight into an FP8 matrix product; the result is
  accumulated in higher precision and returned in 16 bits ("When quantization
  pays", deployment B: a native fp8 GEMM, not a weight-only kernel).

Readings where the pages are silent (listed in the design notes)
----------------------------------------------------------------
F1  The FP8 format is OCP e4m3fn (q_max = 448): sign, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals down to 2^-9, no infinities, the single
    NaN pattern S.1111.111.
F2  Scales are fp32: s = float32(amax) / 448 (IEEE division); the element is
    divided by s in fp32 and the correctly rounded quotient is encoded.
F3  Encoding rounds to the nearest e4m3 value, ties to the even mantissa, and
    saturates to +-448 (the quotient never exceeds 448 by more than rounding).
    The sign of the input is kept, so a negative input that rounds to zero
    encodes as 0x80.
F4  A row or column whose amax is 0 stores scale 0 and all codes 0x00.
F5  Weights are [K, N] with output channel = column n; the scale is taken over
    the K entries of a column.  Activations are [M, K], one scale per row.
F6  Output: Y = s_a[m] * s_w[n] * sum_k dec(qa[m,k]) * dec(qw[k,n]); the oracle
    forms it in fp64.

Native weight order (its own specification; nothing outside fixes it)
--------------------------------------------------------------------
Requires K % 128 == 0 and N % 16 == 0.  KT = K/128, NT = N/16.  The buffer is
N*K bytes in NT*KT tiles of 2048 bytes; tile (nt, kt) starts at byte
(nt*KT + kt)*2048.  Byte lane*32 + i of a tile, lane in [0, 64), i in [0, 32),
is the code of column n = 16*nt + lane%16 at input row
k = 128*kt + 16*(lane//16) + i for i < 16 and k = 128*kt + 64 + 16*(lane//16) + (i-16)
for i >= 16: each 16-byte half of a lane's slot covers 16 consecutive rows, and
the four lane quarters tile 64 consecutive rows per half.
"""
import numpy as np

from .bf16 import bf16_bits_to_f32

QMAX = 448.0


def e4m3_decode_table():
    """Value of every byte 0..255 under OCP e4m3fn, from the format definition (F1)."""
    vals = np.zeros(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9            # subnormal: m/8 * 2^(1-7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS = _TABLE[:127]          # codes 0..126: the non-negative finite values, ascending


def e4m3_decode(codes):
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """fp32 -> e4m3fn code: nearest value, ties to even mantissa, saturate at 448 (F3)."""
    x = np.asarray(x, dtype=np.float32)
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    mag = np.abs(x).astype(np.float64)
    hi = np.searchsorted(_POS, mag, side="left")             # first value >= mag
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - mag
    d_lo = mag - _POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(mag >= _POS[126], 126, code)             # saturation
    code = np.where(mag == 0, 0, code)
    return (code.astype(np.uint8) | (sign << np.uint8(7))).astype(np.uint8)


def _scales(amax):
    """s = amax / 448 in fp32 (F2) and the zero-scale mask of rule F4."""
    s = (amax.astype(np.float32) / np.float32(QMAX)).astype(np.float32)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    return s, zero, s_safe


def quant_act_per_token(a_bits):
    """Dynamic per-token quantization of bf16 activations [M, K] -> (codes [M, K], s [M])."""
    a = bf16_bits_to_f32(a_bits)
    amax = np.max(np.abs(a), axis=1)
    s, zero, s_safe = _scales(amax)
    q = e4m3_encode((a / s_safe[:, None]).astype(np.float32))
    q[zero, :] = 0
    return q, s


def quant_weight_per_channel(w_bits):
    """Per-output-channel quantization of bf16 weights [K, N] -> (codes [K, N], s [N])."""
    w = bf16_bits_to_f32(w_bits)
    amax = np.max(np.abs(w), axis=0)
    s, zero, s_safe = _scales(amax)
    q = e4m3_encode((w / s_safe[None, :]).astype(np.float32))
    q[:, zero] = 0
    return q, s


def pack_native(qw):
    """Native order of the module doc: codes [K, N] -> bytes [N*K]."""
    qw = np.asarray(qw, dtype=np.uint8)
    K, N = qw.shape
    if K % 128 or N % 16:
        raise ValueError("K must be a multiple of 128 and N of 16")
    KT, NT = K // 128, N // 16
    out = np.zeros(N * K, dtype=np.uint8)
    lane = np.arange(64)
    for nt in range(NT):
        cols = 16 * nt + lane % 16
        for kt in range(KT):
            base = (nt * KT + kt) * 2048
            for i in range(32):
                rows = 128 * kt + 64 * (i // 16) + 16 * (lane // 16) + i % 16
                out[base + lane * 32 + i] = qw[rows, cols]
    return out


def unpack_native(buf, K, N):
    buf = np.asarray(buf, dtype=np.uint8)
    KT, NT = K // 128, N // 16
    qw = np.zeros((K, N), dtype=np.uint8)
    lane = np.arange(64)
    for nt in range(NT):
        cols = 16 * nt + lane % 16
        for kt in range(KT):
            base = (nt * KT + kt) * 2048
            for i in range(32):
                rows = 128 * kt + 64 * (i // 16) + 16 * (lane // 16) + i % 16
                qw[rows, cols] = buf[base + lane * 32 + i]
    return qw


def gemm_ref(qa, sa, qw, sw):
    """Y64[m, n] = s_a[m] * s_w[n] * sum_k dec(qa[m, k]) dec(qw[k, n]), in fp64 (F6)."""
    acc = e4m3_decode(qa) @ e4m3_decode(qw)
    return acc * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def gemm_bruteforce(qa, sa, qw, sw):
    """Plain loops over python floats, for tiny shapes only."""
    M, K = qa.shape
    N = qw.shape[1]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(_TABLE[qa[m, k]]) * float(_TABLE[qw[k, n]])
            y[m, n] = acc * float(sa[m]) * float(sw[n])
    return y
