/*
 * qgemm.h -- C ABI of libqgemm.so: the quantized linear layer of LLM decode on
 * AMD Instinct MI355X (gfx950).
 *
 *   W4A16     symmetric INT4 weights, zero offset 8, one bf16 scale per 128
 *             consecutive input rows ("group 128"), bf16 activations, bf16
 *             MFMA with fp32 accumulation, bf16 output.
 *   W8A8-FP8  per-output-channel e4m3 weights with fp32 scales, dynamic
 *             per-token e4m3 activations with fp32 scales, fp8 MFMA with fp32
 *             accumulation, bf16 output.
 *
 * Sources of the operations (page title, then section):
 *   [P1] "When quantization pays -- and when it does not" (mlinterviewnotes,
 *        inference course ch. 04, section 4.4)
 *   [P2] "Give Me BF16 or Give Me Death? Accuracy-Performance Trade-Offs in
 *        LLM Quantization" (paper-graph-ui summary), section 3.4
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Matrices are row-major.  Weights are [K, N] (K = input dimension, the
 * dimension the 128-row groups run along), activations [M, K], outputs
 * [M, N].  bf16 values travel as their uint16 bit patterns.
 *
 * Every pointer argument is a DEVICE pointer (memory the caller allocated on
 * the GPU, e.g. a torch tensor), except where stated.  The library never
 * allocates, frees or keeps a pointer after returning; the caller owns every
 * buffer.  Buffers passed to one call must not overlap unless stated.
 *
 * Every call validates its arguments on the host, synchronously, before it
 * launches anything, and returns:
 *   QG_ERR_NULL       a required pointer is NULL
 *   QG_ERR_SHAPE      M < 0, N <= 0 or K <= 0, K % 128 != 0, N % 16 != 0,
 *                     or a size too large for 32-bit indexing of one matrix
 *                     (shapes are rejected, never padded)
 *   QG_ERR_ALIGN      a matrix pointer is not 16-byte aligned (scale and
 *                     per-row / per-column vectors: 4-byte aligned)
 *   QG_ERR_WORKSPACE  the workspace is smaller than the size query returns
 *   QG_ERR_HIP        the kernel launch itself failed (hipGetLastError)
 * M == 0 is valid and launches nothing.  On success the work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream) and the call returns
 * QG_OK without waiting for it.  Device-side data conditions are not checked:
 * non-finite inputs are outside the contract.
 *
 * Host state: the library keeps per-device caches only (each device's compute
 * unit count and which kernels have their LDS limit raised on it), set
 * idempotently without locks, so calls from several threads and for several
 * devices are safe.  Kernel plans, and with them the workspace sizes, depend
 * on the current device's compute unit count: make a workspace size query
 * with the device current that the call will run on.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_NULL = 1,
    QG_ERR_SHAPE = 2,
    QG_ERR_ALIGN = 3,
    QG_ERR_WORKSPACE = 4,
    QG_ERR_HIP = 5
} qg_status;

/* Opaque stream handle: a hipStream_t. */
typedef void *qg_stream;

/* Static, human-readable text for a status code (host only). */
const char *qg_status_string(int status);

/* Library version string (host only). */
const char *qg_version(void);

/*
 * Size queries (host only, no device access).
 * INT4 g128 storage is K*N/2 bytes of codes plus 2 bytes per group and column:
 * 4.125 bits per weight [P1, opening and "The three regimes"; P2 3.4,
 * "W4A16-INT", group-wise granularity].  Returns 0 for an invalid shape.
 */
size_t qg_int4_g128_packed_bytes(int64_t K, int64_t N);
size_t qg_int4_g128_scale_bytes(int64_t K, int64_t N);

/*
 * Name and configuration of the kernel qgemm_w4a16 / qgemm_w8a8_fp8 launches
 * for this shape on the current device (host only; the text lives in a
 * per-thread buffer valid until the thread's next call; "" for an invalid
 * shape), e.g. "w4a16_decode_kernel<KW, U, D> S=s", "w4a16_small_m_kernel<MT,
 * CT>", "w4a16_large_m_kernel<NS, NB, BM> S=s", "w8a8_small_m_kernel<MT, CT>",
 * "w8a8_large_m_kernel<NS, NB, BM> S=s" (S: K slices across workgroups).
 * Useful to match profiler records to calls.
 */
const char *qg_w4a16_kernel_for(int64_t M, int64_t N, int64_t K);
const char *qg_w8a8_kernel_for(int64_t M, int64_t N, int64_t K);

/* Workspace bytes qgemm_w4a16 / qgemm_w8a8_fp8 need for this shape (may be 0). */
size_t qg_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K);
size_t qg_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * pack_int4_g128 -- offline RTN abs-max INT4 quantization in groups of 128
 * rows, written in the native (MFMA fragment) order.
 * [P2 3.4 "W4A16-INT": s = max|x| / 7 per group of 128 consecutive input-dim
 *  weights, range [-7, 7]; P1 "Counting c": stored code = signed code + 8.]
 *
 *   w_bf16  in   [K, N] bf16 weights.
 *   packed  out  K*N/8 uint32 words (qg_int4_g128_packed_bytes).
 *   scales  out  (K/128)*N bf16 scales (qg_int4_g128_scale_bytes).
 *
 * Per group g and column n: s = bf16_rne(float(amax) / 7.0f); code =
 * clamp(rne(w / s), -8, 7) + 8 with an IEEE fp32 quotient; s == 0 gives
 * code 8 for the whole group.
 *
 * Native order.  G = K/128, NT = N/16.  The words form NT*G tiles of 256
 * words; tile (nt, g) starts at word (nt*G + g)*256.  Word lane*4 + t of a tile
 * (lane < 64, t < 4) holds column n = 16*nt + lane%16 at rows
 * k = 128*g + 32*t + 8*(lane/16) + i, i < 8; nibble slot p (bits 4p..4p+3)
 * holds i = 2p for p < 4 and i = 2(p-4)+1 for p >= 4, so that
 * ((word >> 4j) & 0x000F000F) | 0x43004300 is the bf16 pair
 * (128 + code[2j], 128 + code[2j+1]).  Scale (nt, g, c) sits at
 * (nt*G + g)*16 + c.
 */
qg_status pack_int4_g128(const uint16_t *w_bf16, int K, int N,
                         uint32_t *packed, uint16_t *scales, qg_stream stream);

/*
 * pack_int4_g128_mse -- offline INT4 g128 quantization with MSE-optimal
 * clipping, written in the same native order as pack_int4_g128.
 * [P2 3.4 "W4A16-INT", MSE-optimal clipping: per group the threshold
 *  alpha * max|x|, alpha in (0, 1], that minimizes the summed squared error,
 *  found by grid search; weights beyond it saturate; s = threshold / 7.]
 *
 *   w_bf16   in   [K, N] bf16 weights.
 *   n_alpha  in   grid size: alpha = i / n_alpha, i = 1 .. n_alpha
 *                 (1 <= n_alpha <= 65535; 1 gives the abs-max result).
 *   packed   out  as pack_int4_g128.
 *   scales   out  as pack_int4_g128.
 *
 * Per group g and column n, candidate i has s_i = bf16_rne(float(amax * i) /
 * float(7 * n_alpha)), codes q = clamp(rne(w / s_i), -7, 7) (IEEE fp32
 * quotient; s_i == 0 gives q = 0) and error E_i = sum over the group's rows,
 * in row order, of the fp64 square of w - q * s_i, each square and each
 * partial sum rounded to fp64.  The smallest E_i wins, ties to the larger i;
 * stored code = q + 8.  Cost: n_alpha * 128 fp32 divisions per group.
 */
qg_status pack_int4_g128_mse(const uint16_t *w_bf16, int K, int N, int n_alpha,
                             uint32_t *packed, uint16_t *scales, qg_stream stream);

/*
 * dequant_int4_g128 -- reconstruct the bf16 weights from the native buffers
 * with the same device unpack code the GEMM uses (test / debug export).
 * [P2 3.4 "Inference with W4A16": w_hat = s_g * w_int4; P1 "Counting c": the
 *  offset is removed and the scale applied to the unpacked bf16 pair.]
 *
 *   w_bf16_out  out  [K, N]: bf16_rne((code - 8) * s), the exact fp32 product
 *                    rounded once.
 *   codes_out   out  [K, N] uint8 stored codes (0..15), or NULL to skip.
 */
qg_status dequant_int4_g128(const uint32_t *packed, const uint16_t *scales,
                            int K, int N, uint16_t *w_bf16_out,
                            uint8_t *codes_out, qg_stream stream);

/*
 * qgemm_w4a16 -- y[M, N] = a[M, K] . w_hat[K, N], bf16 in and out, fp32
 * accumulation.
 * [P2 3.4 "Inference with W4A16"; P1 "Counting c" and "The three regimes".]
 *
 *   a_bf16     in   [M, K] activations.
 *   packed     in   native INT4 words from pack_int4_g128.
 *   scales     in   native bf16 scales from pack_int4_g128.
 *   y_bf16     out  [M, N].
 *   workspace  scratch of qg_w4a16_workspace_bytes(M, N, K) bytes (may be
 *              NULL when that is 0), 16-byte aligned.  It must be zero-filled
 *              before its first use.  Its first 64 KiB hold completion
 *              counters (one per output tile or column strip that is split
 *              across workgroups), which every call leaves at zero; the
 *              per-call offset terms and fp32 partial sums follow.  The
 *              counters sit at the same offset for every shape, so one
 *              workspace, sized for the largest call, stays valid for later
 *              calls of any shape.  Calls that share a workspace must not
 *              overlap in time.
 *
 * Numerics (folded offset): the MFMA multiplies the bf16 activations with the
 * exact bf16 values 128 + code; per group and row the kernel adds
 * -136 * sum(a) and multiplies the fp32 group sum by the group scale, i.e. it
 * computes sum_g s_g * sum_{k in g} a_k (code_k - 8) in fp32 -- the product
 * with the exact fp32 dequantized weight -- and rounds the result to bf16.
 */
qg_status qgemm_w4a16(const uint16_t *a_bf16, const uint32_t *packed,
                      const uint16_t *scales, uint16_t *y_bf16,
                      int M, int N, int K,
                      void *workspace, size_t workspace_bytes,
                      qg_stream stream);

/*
 * qgemm_w4a16_noalloc -- qgemm_w4a16 without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops and harnesses that forbid hipMalloc.  It allocates nothing and
 * calls no allocating routine.
 *
 * Same arguments (minus the workspace), kernels, arithmetic and results as
 * qgemm_w4a16.  Its workspace is a library-owned device array of
 * QG_NOALLOC_SCRATCH_BYTES per device (held from the library's load until the
 * process ends): shapes whose qg_w4a16_workspace_bytes exceeds it are rejected
 * with QG_ERR_WORKSPACE before any launch; the array's address on the current
 * device is looked up on the first call there (QG_ERR_HIP if that fails).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (other streams, other threads) race and give undefined
 * results; calls in one stream's order are safe.  The array's completion
 * counters are zero at load and every call leaves them zero.
 */
#define QG_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qg_status qgemm_w4a16_noalloc(const uint16_t *a_bf16, const uint32_t *packed,
                              const uint16_t *scales, uint16_t *y_bf16,
                              int M, int N, int K, qg_stream stream);

/*
 * qgemm_w4a16_grouped -- the W4A16 product of a mixture-of-experts layer: each
 * routed row times its own expert's INT4 g128 weight, bf16 in and out.
 * [P1, the mixture-of-experts section: a batch of B tokens sends about B k / E
 *  rows to each expert, so expert GEMMs stay weight-stream bound far longer
 *  than dense ones; P2 3.4 "Inference with W4A16".]
 *
 *   a_bf16     in   [T, K] routed rows grouped by expert.
 *   offsets    in   device int32 [E + 1]: expert e owns rows
 *                   offsets[e] .. offsets[e+1] - 1 (offsets[0] = 0,
 *                   non-decreasing, offsets[E] = T).
 *   packed     in   E native INT4 weights of [K, N] back to back (expert e at
 *                   word e * K * N / 8), each from pack_int4_g128.
 *   scales     in   the E native scale arrays back to back (expert e at
 *                   element e * (K / 128) * N).
 *   y_bf16     out  [T, N]: row r = a[r] . w_hat_e for the expert e owning r.
 *   E          1 .. 1024.   T   routed rows (0: nothing to do).
 *   workspace  qg_w4a16_grouped_workspace_bytes(E, T, N, K) bytes (4-byte
 *              aligned), no initial contents needed; the size is 0 (NULL is
 *              then accepted) unless the routed rows average 33 or more per
 *              expert that has rows, where it holds the fp32 offset terms of
 *              every routed row.  Calls that share a workspace must not
 *              overlap in time.  The work items (expert, row chunk of up to
 *              16, 32 or 64 rows) are derived on the device by each
 *              workgroup and never stored.
 * Offsets are read on the device and clamped into [0, T] with
 * offsets[e] <= offsets[e+1] enforced per expert, so malformed offsets never
 * cause an access out of bounds; rows they leave unassigned keep their old
 * output, and overlapping ranges give unspecified output rows.
 * QG_ERR_SHAPE: E outside 1 .. 1024, or shapes as qgemm_w4a16 (T as M), or
 * more than 65535 work items (about T / 16 + min(E, T)).
 * Arithmetic per row: exactly that of qgemm_w4a16 for M <= 64 (folded
 * offset, fp32 accumulation).
 */
size_t qg_w4a16_grouped_workspace_bytes(int64_t E, int64_t T, int64_t N, int64_t K);
qg_status qgemm_w4a16_grouped(const uint16_t *a_bf16, const int32_t *offsets,
                              const uint32_t *packed, const uint16_t *scales,
                              uint16_t *y_bf16, int E, int T, int N, int K,
                              void *workspace, size_t workspace_bytes,
                              qg_stream stream);

/*
 * quant_act_per_token -- dynamic per-token e4m3 quantization.
 * [P2 3.4 "W8A8-FP", activation quantization: Q(a_i) = s_i * rnd(a_i / s_i),
 *  s_i = max|a_i| / q_max, computed on the fly per row.]
 *
 *   a_bf16   in   [M, K] activations (K % 128 == 0 is not required here,
 *                 K % 8 == 0 is).
 *   a_e4m3   out  [M, K] OCP e4m3fn codes.
 *   a_scale  out  [M] fp32 scales s = float(amax) / 448.0f (IEEE division).
 * Codes are e4m3(rne(a / s)) of the IEEE fp32 quotient, saturated at +-448;
 * an all-zero row gives s = 0 and codes 0.
 */
qg_status quant_act_per_token(const uint16_t *a_bf16, int M, int K,
                              uint8_t *a_e4m3, float *a_scale, qg_stream stream);

/*
 * quant_weight_fp8_per_channel -- offline per-output-channel e4m3 weight
 * quantization into the native fp8 order.
 * [P2 3.4 "W8A8-FP", weight quantization: per-output-channel symmetric RTN,
 *  s = max|x| / q_max, Q(x) = s * rnd(x / s).]
 *
 *   w_bf16   in   [K, N]; output channel n is column n.
 *   w_e4m3   out  N*K bytes, native order: KT = K/128, NT = N/16 tiles of
 *                 2048 bytes, tile (nt, kt) at byte (nt*KT + kt)*2048; byte
 *                 lane*32 + i (lane < 64, i < 32) is column 16*nt + lane%16 at
 *                 row 128*kt + 64*(i/16) + 16*(lane/16) + i%16.
 *   w_scale  out  [N] fp32, s = float(amax) / 448.0f; zero column -> 0.
 */
qg_status quant_weight_fp8_per_channel(const uint16_t *w_bf16, int K, int N,
                                       uint8_t *w_e4m3, float *w_scale,
                                       qg_stream stream);

/*
 * qgemm_w8a8_fp8 -- y[m, n] = bf16(s_a[m] * s_w[n] * sum_k qa[m,k] qw[k,n])
 * with e4m3 operands on the fp8 MFMA and fp32 accumulation.
 * [P2 3.4 "W8A8-FP"; P1 deployment B: a native fp8 GEMM.]
 *
 *   a_e4m3, a_scale   in  from quant_act_per_token ([M, K], [M]).
 *   w_e4m3, w_scale   in  from quant_weight_fp8_per_channel.
 *   y_bf16            out [M, N].
 *   workspace         scratch of qg_w8a8_workspace_bytes(M, N, K) bytes (NULL
 *                     when that is 0), zero-filled before its first use, with
 *                     the layout and rules of qgemm_w4a16's workspace (64 KiB
 *                     of counters, then fp32 partial sums).
 */
qg_status qgemm_w8a8_fp8(const uint8_t *a_e4m3, const float *a_scale,
                         const uint8_t *w_e4m3, const float *w_scale,
                         uint16_t *y_bf16, int M, int N, int K,
                         void *workspace, size_t workspace_bytes,
                         qg_stream stream);

/*
 * W4A8-FP8 -- INT4 g128 weights (pack_int4_g128's native format) times
 * dynamic per-token e4m3 activations (quant_act_per_token), on the fp8 MFMA.
 * [P1, the mixture-of-experts section: engines pair INT4 weights with FP8
 *  activations on expert layers; P2 3.4 "W4A16-INT" (weights) and "W8A8-FP"
 *  (activations).]
 *
 * y[m, n] = bf16(s_a[m] * sum_g s_g * sum_{k in g} dec(qa[m,k]) (code[k,n] - 8)),
 * fp32 accumulation: each 128-row group is one fp8 MFMA on the codes read as
 * e4m3 bytes (code c is the e4m3 value c * 2^-9) plus the folded offset.
 *
 * qgemm_w4a8_fp8: any M >= 0 (rows in chunks of 16, 32 or 64).
 * qgemm_w4a8_fp8_grouped: rows grouped by expert with device offsets and the
 *   weights and scales of E experts back to back, as qgemm_w4a16_grouped;
 *   a_scale is per routed row.  It needs no workspace: `workspace` and
 *   `workspace_bytes` are not read (NULL and 0 are fine).
 */
qg_status qgemm_w4a8_fp8(const uint8_t *a_e4m3, const float *a_scale,
                         const uint32_t *packed, const uint16_t *scales,
                         uint16_t *y_bf16, int M, int N, int K, qg_stream stream);
qg_status qgemm_w4a8_fp8_grouped(const uint8_t *a_e4m3, const float *a_scale,
                                 const int32_t *offsets, const uint32_t *packed,
                                 const uint16_t *scales, uint16_t *y_bf16,
                                 int E, int T, int N, int K,
                                 void *workspace, size_t workspace_bytes,
                                 qg_stream stream);

/*
 * qgemm_w4a8_fp8_grouped_dynamic -- qgemm_w4a8_fp8_grouped with the per-token
 * e4m3 quantization of the routed rows inside the call: bf16 rows in, the
 * result of quant_act_per_token followed by qgemm_w4a8_fp8_grouped, bit for bit.
 * [P1, the mixture-of-experts section (INT4 expert weights with FP8
 *  activations); P2 3.4 "W8A8-FP" (activation scales computed on the fly).]
 *
 *   a_bf16     in   [T, K] routed rows grouped by expert (as qgemm_w4a16_grouped).
 *   offsets, packed, scales, y_bf16, E, T, N, K: as qgemm_w4a8_fp8_grouped.
 *   workspace  qg_w4a8_grouped_dynamic_workspace_bytes(E, T, N, K) bytes,
 *              16-byte aligned, no initial contents needed: 0 (NULL is then
 *              accepted) when the quantization runs inside the GEMM, else the
 *              codes and scales of the separate quantization.  Calls sharing
 *              it must not overlap in time.
 * With few routed rows (fewer than 48, items of up to 32 rows, K <= 2048; see
 * qg_w4a8_grouped_dynamic_kernel_for) each workgroup quantizes its item's rows
 * into LDS, so no codes reach memory and the call makes one launch fewer.
 * Errors as qgemm_w4a16_grouped (a workspace that is needed but NULL:
 * QG_ERR_NULL; smaller than the query: QG_ERR_WORKSPACE).
 */
size_t qg_w4a8_grouped_dynamic_workspace_bytes(int64_t E, int64_t T, int64_t N, int64_t K);
const char *qg_w4a8_grouped_dynamic_kernel_for(int64_t E, int64_t T, int64_t N, int64_t K);
qg_status qgemm_w4a8_fp8_grouped_dynamic(const uint16_t *a_bf16, const int32_t *offsets,
                                         const uint32_t *packed, const uint16_t *scales,
                                         uint16_t *y_bf16, int E, int T, int N, int K,
                                         void *workspace, size_t workspace_bytes,
                                         qg_stream stream);

/*
 * W8A8-INT8 -- the integer sibling of the fp8 path.
 * [P2 3.4 "W8A8-INT": per-output-channel symmetric weights, s = max|w| / 127,
 *  codes in [-127, 127]; dynamic per-token activations (the scheme the page
 *  uses at 8B and 405B); 8-bit integer product with a 32-bit integer
 *  accumulator, dequantized to 16 bits.]
 *
 * quant_act_per_token_int8: per row m, s_a[m] = float(amax_m) / 127.0f and
 *   q = clamp(rne(a / s_a[m]), -127, 127) with an IEEE fp32 quotient; a zero
 *   row gives s = 0 and codes 0.  K % 8 == 0.
 * quant_weight_int8_per_channel: per column n the same map over the K rows,
 *   written in the fp8 path's native order (quant_weight_fp8_per_channel),
 *   byte for byte.
 * qgemm_w8a8_int8: y[m, n] = bf16(float(sum_k qa[m,k] qw[k,n]) * s_a[m] * s_w[n]),
 *   the sum exact in int32 (K <= 131072, else QG_ERR_SHAPE).  Workspace:
 *   qg_w8a8_int8_workspace_bytes(M, N, K) bytes, zero-filled before first
 *   use, the same layout and rules as qgemm_w8a8_fp8's (int32 slots).
 */
size_t qg_w8a8_int8_workspace_bytes(int64_t M, int64_t N, int64_t K);
qg_status quant_act_per_token_int8(const uint16_t *a_bf16, int M, int K,
                                   int8_t *a_i8, float *a_scale, qg_stream stream);
qg_status quant_weight_int8_per_channel(const uint16_t *w_bf16, int K, int N,
                                        int8_t *w_i8, float *w_scale,
                                        qg_stream stream);
qg_status qgemm_w8a8_int8(const int8_t *a_i8, const float *a_scale,
                          const int8_t *w_i8, const float *w_scale,
                          uint16_t *y_bf16, int M, int N, int K,
                          void *workspace, size_t workspace_bytes,
                          qg_stream stream);

/*
 * qgemm_w8a8_fp8_dynamic / qgemm_w8a8_int8_dynamic -- the W8A8 GEMM with the
 * dynamic per-token activation quantization inside the call: bf16 activations
 * in, y[m, n] = bf16(s_a[m] * s_w[n] * sum_k qa[m,k] qw[k,n]) out, where qa and
 * s_a are exactly what quant_act_per_token (_int8) would produce for a.
 * [P2 3.4 "W8A8-FP" and "W8A8-INT": activation scales computed on the fly per
 *  token; P1 deployment B.]
 *
 *   a_bf16            in  [M, K] activations.
 *   w_e4m3 / w_i8,    in  from quant_weight_fp8_per_channel /
 *   w_scale               quant_weight_int8_per_channel.
 *   y_bf16            out [M, N].
 *   workspace         qg_w8a8_dynamic_workspace_bytes(M, N, K) bytes (NULL
 *                     when that is 0), 16-byte aligned, zero-filled before its
 *                     first use: the GEMM's workspace (the 64 KiB counter
 *                     region first, the rules of qgemm_w8a8_fp8), then the
 *                     codes and scales, always past the counter region, so one
 *                     workspace serves these calls and qgemm_w8a8_fp8 (_int8)
 *                     of any shape in any order.  Calls sharing it must not
 *                     overlap in time.
 *
 * Results equal quant_act_per_token (_int8) followed by qgemm_w8a8_fp8
 * (_int8) bit for bit.  For a few rows (up to four at K = 4096, one at
 * K = 14336; qg_w8a8_dynamic_kernel_for names the choice) each workgroup of
 * the small-M GEMM quantizes the rows itself, into LDS, and no codes reach
 * memory: one launch instead of two; otherwise the codes and scales are
 * written to the workspace by the quantization kernel and read by the GEMM.
 * Errors as qgemm_w8a8_fp8 / qgemm_w8a8_int8.
 */
size_t qg_w8a8_dynamic_workspace_bytes(int64_t M, int64_t N, int64_t K);
const char *qg_w8a8_dynamic_kernel_for(int64_t M, int64_t N, int64_t K);
qg_status qgemm_w8a8_fp8_dynamic(const uint16_t *a_bf16, const uint8_t *w_e4m3,
                                 const float *w_scale, uint16_t *y_bf16,
                                 int M, int N, int K,
                                 void *workspace, size_t workspace_bytes,
                                 qg_stream stream);
qg_status qgemm_w8a8_int8_dynamic(const uint16_t *a_bf16, const int8_t *w_i8,
                                  const float *w_scale, uint16_t *y_bf16,
                                  int M, int N, int K,
                                  void *workspace, size_t workspace_bytes,
                                  qg_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
