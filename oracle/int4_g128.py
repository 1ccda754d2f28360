"""Symmetric INT4, group 128, zero offset 8: the oracle (test infrastructure only).

What the pages fix
------------------
* Scale.  For a group of 128 consecutive weights along the input dimension the
  scale is the group's absolute maximum divided by 7; codes live in [-7, 7] and
  -8 is left unused ("Give Me BF16 or Give Me Death", section 3.4,
  "W4A16-INT Quantization", paragraphs on abs-max clipping and on group-wise
  granularity).
* Storage.  4 bits per weight plus one 16-bit scale per 128 weights, i.e.
  4.125 bits per stored weight ("When quantization pays", opening deployment A
  paragraph and "The three regimes": b_eff = 4.125 bits).
* Zero offset.  The stored nibble is the signed code plus 8 (the unsigned
  4-bit type with bias 8 of the Marlin bf16 path); reconstruction subtracts the
  offset and multiplies by the group scale ("When quantization pays", section
  "Counting c from the kernel, not from intuition").
* Product.  Y = X . W_hat with W_hat = s_g * w_int4, 16-bit activations and a
  higher-precision accumulator ("Give Me BF16", section 3.4, "Inference with
  W4A16").

Readings where the pages are silent (each is listed in the design notes)
-----------------------------------------------------------------------
R1  The scale is stored in bf16 (the pages' kernel works on bf16 pairs; the
    second page's "FP16" is read as the 16-bit type of the activations).
R2  Codes are computed by dividing by the *stored* bf16 scale, so that
    quantization and reconstruction use the same number.
R3  rnd() is round-half-to-even applied to the correctly rounded fp32
    quotient; the code is clamped to [-8, 7] (abs-max never reaches -8, but
    the clamp makes the map total, and dequantization accepts code 0 -> -8).
R4  A group whose bf16 scale is zero (all-zero group, or amax/7 below half the
    smallest bf16 subnormal) stores scale 0 and code 8 everywhere.
R5  Layouts: weights are [K, N] (K = input dimension, groups run along K);
    activations are [M, K]; outputs are [M, N].

Native order (the MFMA fragment order; its own specification, nothing outside
fixes it, so its parity is "unpinned" beyond this text)
------------------------------------------------------
Requires K % 128 == 0 and N % 16 == 0.  G = K/128 groups, NT = N/16 column
tiles.  The packed buffer is K*N/8 uint32 words made of NT*G tiles of 256
words (1 KiB); tile (nt, g) starts at word (nt*G + g)*256.  Word
(lane, t) of a tile, lane in [0, 64), t in [0, 4), sits at lane*4 + t and holds
the eight codes of column n = 16*nt + lane%16 at input rows
k = 128*g + 32*t + 8*(lane//16) + i, i in [0, 8): word t feeds MFMA k-step t,
whose 32 rows the four lane quarters split into consecutive 8-row pieces.  Nibble slot p (bits 4p..4p+3)
holds row offset i = SLOT_TO_ROW[p] = (0, 2, 4, 6, 1, 3, 5, 7)[p], so that
slots p and p+4 hold the consecutive rows (2p, 2p+1).
The native scales are NT*G*16 bf16 values; entry (nt, g, c) at
(nt*G + g)*16 + c is the scale of group g of column 16*nt + c.
"""
import numpy as np

from .bf16 import bf16_bits_to_f32, f32_to_bf16_bits

GROUP = 128
OFFSET = 8
SLOT_TO_ROW = (0, 2, 4, 6, 1, 3, 5, 7)


def _check_shape(K, N, need_tile=True):
    if K % GROUP:
        raise ValueError(f"K={K} is not a multiple of the group size {GROUP}")
    if need_tile and N % 16:
        raise ValueError(f"N={N} is not a multiple of 16")


def quantize(w_bits):
    """RTN abs-max INT4 quantization in groups of 128 rows along K.

    w_bits: uint16 bf16 patterns [K, N].
    Returns (codes uint8 [K, N] in [0, 15], scale_bits uint16 [K/128, N]).
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K, N = w_bits.shape
    _check_shape(K, N, need_tile=False)
    G = K // GROUP
    w = bf16_bits_to_f32(w_bits).reshape(G, GROUP, N)
    # step 1: the group's absolute maximum (exact: the inputs are bf16)
    amax = np.max(np.abs(w), axis=1)                            # [G, N] fp32
    # step 2: s = amax / 7 in fp32, stored as bf16 (reading R1)
    s_bits = f32_to_bf16_bits(amax / np.float32(7.0))           # [G, N]
    s = bf16_bits_to_f32(s_bits)
    # step 3: code = clamp(rne(w / s), -8, 7) + 8 (readings R2, R3, R4)
    zero = s == 0
    s_safe = np.where(zero, np.float32(1.0), s)
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.rint(w / s_safe[:, None, :])                     # fp32 quotient, then half-even
    q = np.clip(q, -8, 7)
    q = np.where(zero[:, None, :], 0.0, q)
    codes = (q.astype(np.int16) + OFFSET).astype(np.uint8).reshape(K, N)
    return codes, s_bits


def quantize_mse(w_bits, n_alpha=100):
    """INT4 g128 quantization with MSE-optimal clipping, searched on a grid.

    "Give Me BF16 or Give Me Death", section 3.4, "W4A16-INT", paragraphs on
    MSE-optimal clipping: per group of 128 weights, instead of the abs-max
    range the clipping threshold is alpha * max|x| with alpha in (0, 1], the
    scale is that threshold over 7, weights beyond the threshold saturate at
    the largest code, and alpha minimizes the group's summed squared error
    sum_i (x_i - Q_alpha(x_i))^2, found by a grid search over the scalar.

    Readings where the page is silent (listed with the design notes):
    M1  The grid is alpha_i = i / n_alpha, i = 1 .. n_alpha (default 100
        uniform steps); among equal errors the larger alpha wins.
    M2  The candidate scale is bf16_rne(float32(amax * i) / float32(7 * n_alpha)):
        amax * i is exact in fp32 (an 8-bit bf16 mantissa times an integer
        below 2^16) and the division is one IEEE fp32 quotient, so i = n_alpha
        reproduces the abs-max scale of quantize() exactly.
    M3  Codes are clamp(rne(x / s), -7, 7) with the IEEE fp32 quotient (the
        page's symmetric range; saturation is the clipping), scale 0 gives
        code 0; stored code = code + 8.
    M4  The error is evaluated in fp64: d = x - q * s (exact), then the 128
        squares d * d are each rounded to fp64 and added in row order, one
        rounding per addition.

    w_bits: uint16 bf16 patterns [K, N].  Returns (codes uint8 [K, N],
    scale_bits uint16 [K/128, N]) like quantize().
    """
    if not 1 <= n_alpha <= 65535:
        raise ValueError(f"n_alpha={n_alpha} outside [1, 65535]")
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K, N = w_bits.shape
    _check_shape(K, N, need_tile=False)
    G = K // GROUP
    w = bf16_bits_to_f32(w_bits).reshape(G, GROUP, N)
    w64 = w.astype(np.float64)
    amax = np.max(np.abs(w), axis=1)                            # [G, N] fp32, exact

    def codes_for(s):
        zero = s == 0
        s_safe = np.where(zero, np.float32(1.0), s)
        with np.errstate(over="ignore", invalid="ignore"):
            q = np.rint(w / s_safe[:, None, :])                 # fp32 quotient, then half-even
        q = np.clip(q, -7, 7)                                   # saturate beyond the threshold
        return np.where(zero[:, None, :], 0.0, q)

    best_err = np.full((G, N), np.inf)
    best_bits = np.zeros((G, N), dtype=np.uint16)
    for i in range(1, n_alpha + 1):
        with np.errstate(over="ignore"):
            t = amax * np.float32(i)                             # exact (reading M2)
            s_bits = f32_to_bf16_bits(t / np.float32(7 * n_alpha))
        s = bf16_bits_to_f32(s_bits)
        q = codes_for(s).astype(np.float64)
        s64 = s.astype(np.float64)
        err = np.zeros((G, N))
        with np.errstate(invalid="ignore", over="ignore"):
            for j in range(GROUP):                              # row order (reading M4)
                d = w64[:, j, :] - q[:, j, :] * s64
                err = err + d * d
        take = err <= best_err                                  # ties: the larger alpha
        best_err = np.where(take, err, best_err)
        best_bits = np.where(take, s_bits, best_bits)
    q = codes_for(bf16_bits_to_f32(best_bits))
    codes = (q.astype(np.int16) + OFFSET).astype(np.uint8).reshape(K, N)
    return codes, best_bits


def group_sq_error(w_bits, codes, scale_bits):
    """sum over each group of (x - (code - 8) * s)^2 in fp64, [K/128, N]."""
    K, N = codes.shape
    x = bf16_bits_to_f32(w_bits).astype(np.float64)
    d = x - dequant_f32(codes, scale_bits).astype(np.float64)
    return (d * d).reshape(K // GROUP, GROUP, N).sum(axis=1)


def dequant_f32(codes, scale_bits):
    """w_hat = (code - 8) * s in fp32.  Exact: at most 4 + 8 significant bits."""
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    s = bf16_bits_to_f32(scale_bits)                            # [G, N]
    q = codes.astype(np.float32) - np.float32(OFFSET)
    with np.errstate(over="ignore"):
        return (q.reshape(K // GROUP, GROUP, N) * s[:, None, :]).reshape(K, N)


def dequant_bf16_bits(codes, scale_bits):
    """The bf16 value a 16-bit MMA operand holds: RNE of the exact product.

    Equal to the page's kernel semantics: the offset subtraction on the
    bf16 pair is exact, and the one bf16 multiply by the scale rounds the exact
    product once.
    """
    return f32_to_bf16_bits(dequant_f32(codes, scale_bits))


def stored_bytes(K, N):
    """Bytes stored for a [K, N] INT4 g128 weight: K*N/2 codes + 2 bytes per group."""
    return K * N // 2 + 2 * N * (K // GROUP)


def pack_canonical(codes):
    """Plain packing: uint32 [K/8, N]; code of row k = 8j + i in bits 4i..4i+3 of word (j, n)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        words |= codes[i::8, :].astype(np.uint32) << np.uint32(4 * i)
    return words


def pack_native(codes, scale_bits):
    """Native (MFMA fragment) order, written from the specification in the module doc.

    Returns (packed uint32 [K*N/8], scales uint16 [NT*G*16]).
    """
    codes = np.asarray(codes, dtype=np.uint8)
    K, N = codes.shape
    _check_shape(K, N)
    G, NT = K // GROUP, N // 16
    packed = np.zeros(NT * G * 256, dtype=np.uint32)
    lane = np.arange(64)
    for nt in range(NT):
        cols = 16 * nt + lane % 16                               # [64]
        for g in range(G):
            base = (nt * G + g) * 256
            for t in range(4):
                kb = GROUP * g + 32 * t + 8 * (lane // 16)       # [64]
                word = np.zeros(64, dtype=np.uint32)
                for p in range(8):
                    code = codes[kb + SLOT_TO_ROW[p], cols].astype(np.uint32)
                    word |= code << np.uint32(4 * p)
                packed[base + lane * 4 + t] = word
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    scales = np.zeros(NT * G * 16, dtype=np.uint16)
    for nt in range(NT):
        for g in range(G):
            scales[(nt * G + g) * 16:(nt * G + g + 1) * 16] = scale_bits[g, 16 * nt:16 * nt + 16]
    return packed, scales


def unpack_native(packed, scales, K, N):
    """Inverse of pack_native: (codes uint8 [K, N], scale_bits uint16 [K/128, N])."""
    _check_shape(K, N)
    G, NT = K // GROUP, N // 16
    packed = np.asarray(packed, dtype=np.uint32)
    codes = np.zeros((K, N), dtype=np.uint8)
    lane = np.arange(64)
    for nt in range(NT):
        cols = 16 * nt + lane % 16
        for g in range(G):
            base = (nt * G + g) * 256
            for t in range(4):
                kb = GROUP * g + 32 * t + 8 * (lane // 16)
                word = packed[base + lane * 4 + t]
                for p in range(8):
                    codes[kb + SLOT_TO_ROW[p], cols] = (word >> np.uint32(4 * p)) & np.uint32(0xF)
    scales = np.asarray(scales, dtype=np.uint16)
    scale_bits = np.zeros((G, N), dtype=np.uint16)
    for nt in range(NT):
        for g in range(G):
            scale_bits[g, 16 * nt:16 * nt + 16] = scales[(nt * G + g) * 16:(nt * G + g + 1) * 16]
    return codes, scale_bits


def gemm_ref(a_bits, codes, scale_bits):
    """Y64 = float64(A) @ float64(w_hat_fp32): the W4A16 product in fp64.

    a_bits: bf16 patterns [M, K]; codes/scale_bits as returned by quantize().
    """
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    w = dequant_f32(codes, scale_bits).astype(np.float64)
    return a @ w


def grouped_gemm_ref(a_bits, offsets, experts):
    """The expert-grouped W4A16 product in fp64.

    A mixture-of-experts layer sends each routed row through its own expert's
    weight ("When quantization pays", the mixture-of-experts section: a batch
    of B tokens gives every expert about B k / E rows).  Rows are grouped by
    expert: expert e owns rows offsets[e] .. offsets[e+1]-1 of a_bits [T, K],
    and its output rows are those rows times that expert's dequantized weight.

    experts: {e: (codes, scale_bits)} as returned by quantize(); only the
    listed experts are computed.  Returns {e: Y64 [rows_e, N]}.
    """
    out = {}
    for e, (codes, s) in experts.items():
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        out[e] = gemm_ref(a_bits[r0:r1], codes, s)
    return out


def gemm_ref_bf16_operand(a_bits, codes, scale_bits):
    """Diagnostic variant: the product with the bf16-rounded dequantized operand."""
    a = bf16_bits_to_f32(a_bits).astype(np.float64)
    w = bf16_bits_to_f32(dequant_bf16_bits(codes, scale_bits)).astype(np.float64)
    return a @ w


def gemm_bruteforce(a_bits, codes, scale_bits):
    """Plain triple loop over python floats, for tiny shapes only."""
    a = bf16_bits_to_f32(a_bits)
    s = bf16_bits_to_f32(scale_bits)
    M, K = a.shape
    N = codes.shape[1]
    y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(a[m, k]) * ((int(codes[k, n]) - 8) * float(s[k // GROUP, n]))
            y[m][n] = acc
    return np.array(y, dtype=np.float64)
