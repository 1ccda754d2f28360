// W4A8-FP8 on gfx950: INT4 g128 weights (the W4A16 native format) times
// dynamic per-token e4m3 activations on the fp8 MFMA.
//
// "When quantization pays", mixture-of-experts section: serving engines pair
// INT4 weights with FP8 activations on the expert layers.  The weight format is
// that of "Give Me BF16 or Give Me Death" section 3.4 "W4A16-INT", the
// activation quantization that of its "W8A8-FP" paragraph.
//
// A 4-bit code c (0..15) read as an OCP e4m3 byte is exactly c * 2^-9 (0x00-0x07
// are the subnormals m * 2^-9, 0x08-0x0F the lowest binade), so a native word
// becomes two MFMA operand dwords with two ANDs: w & 0x0F0F0F0F holds the codes
// of nibble slots 0, 2, 4, 6 and (w >> 4) & 0x0F0F0F0F those of slots 1, 3, 5,
// 7, one per byte.  A 128-row group is one 16x16x128 fp8 MFMA.  The offset is
// folded as in W4A16: the group's accumulator starts at A . (-8 * 2^-9) (an
// MFMA against the constant byte 0x88), so the group sum is
// 2^-9 * sum_k dec(qa_k) (c_k - 8); it is scaled by 512 * s_g into the fp32
// total, and the epilogue multiplies by s_a[m].
//
// Byte pairing: for word t (rows 32t + 8q .. +7 of the group, q = lane / 16) the
// B bytes are the slots (0, 2, 4, 6 | 1, 3, 5, 7), i.e. rows (0, 4, 1, 5 | 2, 6,
// 3, 7); the A fragment of the same lane loads its row's 8 activation bytes at
// k = 32t + 8q and permutes them into that order (two v_perm_b32), so A and B
// hold the same k in every byte position whatever order the MFMA sums in.

#include "device_common.h"
#include "launch.h"

namespace qg {

template <int MT, int CT, int NWAVE>
__device__ __forceinline__ void w4a8_tile(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                          const uint32_t* __restrict__ wq,
                                          const uint16_t* __restrict__ sc, uint16_t* __restrict__ y,
                                          int M, int N, int K, int nt0) {
    const int G = K >> 7;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15;
    const int q = lane >> 4;
    const int g_begin = (G * wave) / NWAVE;
    const int g_end = (G * (wave + 1)) / NWAVE;

    f32x4 total[CT][MT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) total[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint8_t* arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        arow[mt] = qa + (size_t)min(mt * 16 + col, M - 1) * K + 8 * q;   // rows >= M: discarded
    const u32x4* wp[CT];
    const uint16_t* sp[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const size_t tile = (size_t)(nt0 + ct) * G;
        wp[ct] = reinterpret_cast<const u32x4*>(wq) + tile * 64 + lane;
        sp[ct] = sc + tile * 16 + col;
    }
    i32x8 neg8;                                    // e4m3 0x88 = -8 * 2^-9 in every byte
#pragma unroll
    for (int i = 0; i < 8; ++i) neg8[i] = (int)0x88888888u;

    struct Buf {
        uint2 a[MT][4];
        u32x4 w[CT];
        uint32_t s[CT];
    };
    auto load = [&](int g, Buf& b) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            b.w[ct] = __builtin_nontemporal_load(wp[ct] + (size_t)g * 64);
            b.s[ct] = sp[ct][(size_t)g * 16];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                b.a[mt][t] = *reinterpret_cast<const uint2*>(arow[mt] + (size_t)g * 128 + 32 * t);
    };
    auto compute = [&](const Buf& b) {
        i32x8 af[MT];
        f32x4 corr[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[mt][2 * t] = (int)__builtin_amdgcn_perm(b.a[mt][t].y, b.a[mt][t].x, 0x05010400u);
                af[mt][2 * t + 1] = (int)__builtin_amdgcn_perm(b.a[mt][t].y, b.a[mt][t].x, 0x07030602u);
            }
            corr[mt] = mfma_fp8_16x16x128(af[mt], neg8, f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint32_t wd[4] = {b.w[ct].x, b.w[ct].y, b.w[ct].z, b.w[ct].w};
            i32x8 bf;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                bf[2 * t] = (int)(wd[t] & 0x0F0F0F0Fu);
                bf[2 * t + 1] = (int)((wd[t] >> 4) & 0x0F0F0F0Fu);
            }
            const float s = bf16_to_f32(b.s[ct]) * 512.0f;          // exact: 2^9 s_g
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 acc = mfma_fp8_16x16x128(af[mt], bf, corr[mt]);
#pragma unroll
                for (int i = 0; i < 4; ++i) total[ct][mt][i] = fmaf(s, acc[i], total[ct][mt][i]);
            }
        }
    };

    // two buffers, unrolled by two; the load past the range repeats the last
    // group (never computed), so every load is unconditional
    Buf b0, b1;
    if (g_begin < g_end) load(g_begin, b0);
    int g = g_begin;
    for (; g + 1 < g_end; g += 2) {
        load(g + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0);
        load(min(g + 2, g_end - 1), b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(b1);
    }
    if (g < g_end) compute(b0);

    __shared__ f32x4 red[NWAVE][CT][MT][64];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wave][ct][mt][lane] = total[ct][mt];
    __syncthreads();
    for (int e = threadIdx.x; e < CT * MT * 256; e += NWAVE * 64) {
        const int i = e & 3;
        const int l = (e >> 2) & 63;
        const int cm = e >> 8;
        const int mt = cm % MT;
        const int ct = cm / MT;
        const int m = mt * 16 + 4 * (l >> 4) + i;
        if (m >= M) continue;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) sum += red[w][ct][mt][l][i];
        const int n = (nt0 + ct) * 16 + (l & 15);
        y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(sum * sa[m]);
    }
}

// dense: blockIdx.y takes rows [16 MT y, 16 MT (y + 1))
template <int MT, int CT, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) void w4a8_kernel(const uint8_t* __restrict__ qa,
                                                          const float* __restrict__ sa,
                                                          const uint32_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ sc,
                                                          uint16_t* __restrict__ y, int M, int N, int K) {
    const int row0 = blockIdx.y * 16 * MT;
    w4a8_tile<MT, CT, NWAVE>(qa + (size_t)row0 * K, sa + row0, wq, sc, y + (size_t)row0 * N,
                             min(16 * MT, M - row0), N, K, blockIdx.x * CT);
}

// expert-grouped: one work item (expert, first row, rows) of the W4A16 grouped
// path's item list per blockIdx.y
template <int MT, int CT, int NWAVE>
__global__ __launch_bounds__(NWAVE * 64) void w4a8_grouped_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const int* __restrict__ items,
    const uint32_t* __restrict__ wq, const uint16_t* __restrict__ sc, uint16_t* __restrict__ y,
    int N, int K) {
    const int it = blockIdx.y;
    if (it >= items[0]) return;
    const int e = items[1 + 3 * it];
    const int r0 = items[2 + 3 * it];
    const int rows = items[3 + 3 * it];
    const size_t words = (size_t)(K / 8) * N;
    const size_t nsc = (size_t)(K / 128) * N;
    w4a8_tile<MT, CT, NWAVE>(qa + (size_t)r0 * K, sa + r0, wq + e * words, sc + e * nsc,
                             y + (size_t)r0 * N, rows, N, K, blockIdx.x * CT);
}

constexpr int W4A8_NWAVE = 4;
#ifndef QG_W4A8_ONE_WAVE_MIN_T     // grouped: one wave per workgroup from this many routed rows
#define QG_W4A8_ONE_WAVE_MIN_T 128
#endif

static int w4a8_ct(int NT) { return NT % 4 == 0 ? 4 : (NT % 2 == 0 ? 2 : 1); }

template <class F>
static void w4a8_dispatch(int MT, int CT, F&& f) {
    auto by_ct = [&](auto mt) {
        if (CT == 4) f(mt, ic<4>{});
        else if (CT == 2) f(mt, ic<2>{});
        else f(mt, ic<1>{});
    };
    if (MT == 1) by_ct(ic<1>{});
    else if (MT == 2) by_ct(ic<2>{});
    else by_ct(ic<4>{});
}

void launch_qgemm_w4a8_fp8(const uint8_t* qa, const float* sa, const uint32_t* wq,
                           const uint16_t* sc, uint16_t* y, int M, int N, int K, hipStream_t s) {
    const int MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    const int NT = N / 16;
    const int CT = w4a8_ct(NT);
    const dim3 grid(NT / CT, (M + 16 * MT - 1) / (16 * MT));
    w4a8_dispatch(MT, CT, [&](auto mt, auto ct) {
        hipLaunchKernelGGL((w4a8_kernel<decltype(mt)::value, decltype(ct)::value, W4A8_NWAVE>), grid,
                           dim3(W4A8_NWAVE * 64), 0, s, qa, sa, wq, sc, y, M, N, K);
    });
}

void launch_qgemm_w4a8_fp8_grouped(const uint8_t* qa, const float* sa, const int* offsets,
                                   const uint32_t* wq, const uint16_t* sc, uint16_t* y, int E, int T,
                                   int N, int K, void* ws, hipStream_t s) {
    const int R = w4a16_grouped_rows_per_item(E, T);
    const int max_items = w4a16_grouped_max_items(E, T);
    int* items = static_cast<int*>(ws);
    launch_grouped_items(offsets, E, T, R, max_items, items, s);
    const int NT = N / 16;
    const int CT = w4a8_ct(NT);
    if (T >= QG_W4A8_ONE_WAVE_MIN_T) {
        // many routed rows: one wave per workgroup over the whole K (no K split,
        // no LDS reduction) and many more workgroups in flight; measured at top-8
        // over 128 experts: B = 16 / 64 / 1024 -4 / -8 / -27 % (B = 1, with a
        // handful of workgroups, is 26 % slower this way)
        w4a8_dispatch(R / 16, CT, [&](auto mt, auto ct) {
            hipLaunchKernelGGL((w4a8_grouped_kernel<decltype(mt)::value, decltype(ct)::value, 1>),
                               dim3(NT / decltype(ct)::value, max_items), dim3(64), 0, s, qa, sa, items, wq,
                               sc, y, N, K);
        });
        return;
    }
    w4a8_dispatch(R / 16, CT, [&](auto mt, auto ct) {
        hipLaunchKernelGGL((w4a8_grouped_kernel<decltype(mt)::value, decltype(ct)::value, W4A8_NWAVE>),
                           dim3(NT / decltype(ct)::value, max_items), dim3(W4A8_NWAVE * 64), 0, s, qa, sa,
                           items, wq, sc, y, N, K);
    });
}

}  // namespace qg
