// Chained decode: the W4A16 GEMMs of one decode step (M <= 16) in one
// persistent, cooperative launch.
//
// One workgroup per compute unit, all resident at once (a cooperative launch
// either guarantees that or fails to launch).  For GEMM i every workgroup owns
// at most one strip of column tiles ("unit"); the strips split the columns as
// evenly as the tile count allows.  Inside a workgroup the 8 waves are kw
// K-sub-ranges x 8/kw tile slots (kw > 1 when a strip has few tiles: the
// narrow projections), and a wave streams (tile, U-group chunk) items of its
// share through a register prefetch loop, exactly as in the single-GEMM decode
// kernel: activations and the -136 * sum(a) offset terms staged in LDS, the
// unpacked weights fed to bf16 MFMA, per-group scales applied on the fp32 sums.
// When a[M, K] does not fit in LDS, K is processed in chunks that do.
//
// Dependencies.  A GEMM flagged "after previous" reads memory the previous
// GEMM writes (in a model, its input is the previous output).  Each workgroup
// issues the loads of its first weight item, then waits until every
// workgroup has finished the previous GEMM (a counter per GEMM), so the weight
// stream keeps flowing across the boundary.  Outputs are written, and
// activations read, with agent-scope atomic accesses, which are coherent
// across the XCDs' separate L2 caches without cache-wide maintenance.  The wait
// is bounded: past the limit it sets the error word and proceeds, so every
// wave always exits.  The last workgroup to finish resets all counters.

#include "device_common.h"
#include "launch.h"

namespace qg {

constexpr int CH_NWAVE = 8;
constexpr unsigned CH_SPIN_LIMIT = 1u << 24;

__device__ __forceinline__ u32x4 load_coherent_b128(const void* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    u32x4 r;
    r.x = (uint32_t)lo;
    r.y = (uint32_t)(lo >> 32);
    r.z = (uint32_t)hi;
    r.w = (uint32_t)(hi >> 32);
    return r;
}

__device__ __forceinline__ void store_coherent_u16(uint16_t* p, uint32_t v) {
    __hip_atomic_store(p, (uint16_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int U>
__device__ void chain_gemm(const ChainDesc& d, int M, unsigned char* lds, unsigned* done_prev,
                           unsigned* err, int P) {
    const int N = d.N;
    const int K = d.K;
    const int G = K >> 7;
    const int NT = N >> 4;
    const int kw = d.kw;
    const int TW = CH_NWAVE / kw;
    const int nch = d.nchunks;
    const int Gc = G / nch;                       // groups per K-chunk
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;

    const int unit = blockIdx.x;
    const bool has = unit < d.units;
    const int t0 = has ? (int)(((long long)NT * unit) / d.units) : 0;
    const int t1 = has ? (int)(((long long)NT * (unit + 1)) / d.units) : 0;
    const int ksub = wave % kw;
    const int tslot = wave / kw;
    const int ng = Gc / kw;                       // groups per wave per chunk
    const int nq = ng / U;                        // items per tile per chunk
    const int ntiles = has && t1 - t0 > tslot ? (t1 - t0 - tslot + TW - 1) / TW : 0;
    const int ipc = ntiles * nq;                  // items per chunk (this wave)
    const int nitems = ipc * nch;

    const int rowb = Gc * 256 + 16;
    float* corr = reinterpret_cast<float*>(lds + (size_t)M * rowb);      // [Gc][16]
    float* red = corr + Gc * 16;                                           // [T][kw][256]

    // item -> (chunk, tile slot j, chunk q); first group of the item within K
    auto item_tile = [&](int it) { return t0 + tslot + ((it % ipc) / nq) * TW; };
    auto item_g0 = [&](int it) {
        return (it / ipc) * Gc + ksub * ng + ((it % ipc) % nq) * U;
    };

    const int slane = lane % (8 * U);
    // item i lives in buffer i & 1 (no register copies: a copy of a register
    // with a load in flight would wait for that load and drain the pipeline)
    u32x4 wa[U], wb[U];
    uint32_t sa = 0, sb = 0;
    auto load_item = [&](int it, u32x4 (&w)[U], uint32_t& sv) {
        const size_t tile0 = (size_t)item_tile(it) * G + item_g0(it);   // wave-uniform
        const u32x4* wp = reinterpret_cast<const u32x4*>(d.wq) + tile0 * 64;
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(wp + u * 64 + lane);
        sv = reinterpret_cast<const uint32_t*>(d.sc + tile0 * 16)[slane];
    };
    if (nitems > 0) load_item(0, wa, sa);         // weights first: they depend on nothing

    if (d.after_prev) {                            // wait for the previous GEMM
        if (tid == 0) {
            unsigned spins = 0;
            while (__hip_atomic_load(done_prev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   (unsigned)P) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > CH_SPIN_LIMIT) {
                    __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
    }

    const Int4Unpacker unpack;
    const int sidx = (col >> 1) << 2;
    const int shalf = (col & 1) << 4;
    const unsigned char* arow = lds + (size_t)min(col, M - 1) * rowb + kq * 16;
    const float* crow = corr + 4 * kq;
    f32x4 total = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_item = [&](int it, const u32x4 (&w)[U], uint32_t sv) {
        const int gl0 = item_g0(it) - (it / ipc) * Gc;      // group within the chunk
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = gl0 + u;
            f32x4 acc = *reinterpret_cast<const f32x4*>(crow + g * 16);
            const uint32_t pair = (uint32_t)__builtin_amdgcn_ds_bpermute(sidx + u * 32, (int)sv);
            const float s = bf16_to_f32((pair >> shalf) & 0xffffu);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(arow + g * 256 + t * 64));
                const uint32_t wv = t == 0 ? w[u].x : t == 1 ? w[u].y : t == 2 ? w[u].z : w[u].w;
                acc = mfma_bf16_16x16x32(af, unpack(wv), acc);
            }
            total[0] = fmaf(s, acc[0], total[0]);
            total[1] = fmaf(s, acc[1], total[1]);
            total[2] = fmaf(s, acc[2], total[2]);
            total[3] = fmaf(s, acc[3], total[3]);
        }
        if ((it % ipc) % nq == nq - 1 && it / ipc == nch - 1) {   // tile complete
            const int tile = item_tile(it);
            if (kw == 1) {
                const int n = tile * 16 + col;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * kq + i;
                    if (m < M) store_coherent_u16(d.y + (size_t)m * N + n, f32_to_bf16_rne(total[i]));
                }
            } else {
                *reinterpret_cast<f32x4*>(red + ((tile - t0) * kw + ksub) * 256 + lane * 4) = total;
            }
            total = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    int it = 0;
    for (int c = 0; c < nch; ++c) {
        if (has) {                                 // stage a[:, chunk c] and its offset terms
            const int cpr = Gc * 16;
            const int tot = M * cpr;
            const size_t kofs = (size_t)c * Gc * 128;
            for (int e = tid; e < tot; e += CH_NWAVE * 64) {
                const int r = e / cpr;
                const int cc = e - r * cpr;
                const u32x4 v = load_coherent_b128(d.a + (size_t)r * K + kofs + (size_t)cc * 8);
                *reinterpret_cast<u32x4*>(lds + (size_t)r * rowb + cc * 16) = v;
            }
            __syncthreads();
            // the offset terms exactly as the single-GEMM decode kernel forms them
            decode_offset_terms(lds, rowb, corr, lds + (size_t)min(col, M - 1) * rowb + kq * 16, M, Gc, tid,
                                wave, col, kq, CH_NWAVE);
            __syncthreads();
        }
        // this chunk's items: each step prefetches the wave's next item (which
        // may lie in the next chunk) into the other buffer, then computes; the
        // wave's very last item is peeled off so every prefetch is unconditional
        const int end = min((c + 1) * ipc, nitems - 1);
        for (; it < end; ++it) {
            if ((it & 1) == 0) {
                load_item(it + 1, wb, sb);
                __builtin_amdgcn_sched_barrier(0);
                compute_item(it, wa, sa);
            } else {
                load_item(it + 1, wa, sa);
                __builtin_amdgcn_sched_barrier(0);
                compute_item(it, wb, sb);
            }
        }
        if (it == nitems - 1 && it < (c + 1) * ipc) {
            if ((it & 1) == 0)
                compute_item(it, wa, sa);
            else
                compute_item(it, wb, sb);
            ++it;
        }
        if (has) __syncthreads();                  // before the next chunk overwrites LDS
    }

    if (has && kw > 1) {                           // add the kw partial sums of each tile
        const int T = t1 - t0;
        for (int e = tid; e < T * 256; e += CH_NWAVE * 64) {
            const int tl = e >> 8;
            const int r = e & 255;
            float v = 0.0f;
            for (int k = 0; k < kw; ++k) v += red[(tl * kw + k) * 256 + r];
            const int m = 4 * ((r >> 2) >> 4) + (r & 3);
            const int n = (t0 + tl) * 16 + ((r >> 2) & 15);
            if (m < M) store_coherent_u16(d.y + (size_t)m * N + n, f32_to_bf16_rne(v));
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(CH_NWAVE * 64) void w4a16_chain_kernel(const ChainDesc* __restrict__ plan,
                                                                    int count, int M,
                                                                    unsigned* __restrict__ ws) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned* exit_count = ws;
    unsigned* err = ws + 1;
    unsigned* done = ws + 2;
    const int P = gridDim.x;
    for (int i = 0; i < count; ++i) {
        const ChainDesc d = plan[i];
        unsigned* done_prev = i > 0 ? done + i - 1 : done;
        switch (d.u) {
            case 8: chain_gemm<8>(d, M, lds, done_prev, err, P); break;
            case 4: chain_gemm<4>(d, M, lds, done_prev, err, P); break;
            case 2: chain_gemm<2>(d, M, lds, done_prev, err, P); break;
            default: chain_gemm<1>(d, M, lds, done_prev, err, P); break;
        }
        // this workgroup's outputs of GEMM i are complete before it is counted
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(done + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {                        // the last workgroup out resets the counters
        const unsigned prev =
            __hip_atomic_fetch_add(exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)P - 1) {
            for (int i = 0; i < count; ++i)
                __hip_atomic_store(done + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(exit_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: planning and launch
// ---------------------------------------------------------------------------
#ifndef QG_CH_LDS_BUDGET
#define QG_CH_LDS_BUDGET (144 * 1024)
#endif

static int chain_cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}

int chain_grid() { return chain_cu_count(); }

static size_t chain_lds(int M, int Gc, int tmax, int kw) {
    return (size_t)M * (Gc * 256 + 16) + (size_t)Gc * 16 * sizeof(float) +
           (kw > 1 ? (size_t)tmax * kw * 256 * sizeof(float) : 0);
}

static int chain_u(int ng) {
    for (int u : {8, 4, 2, 1})
        if (ng % u == 0) return u;
    return 1;
}

bool chain_plan_one(int M, int N, int K, int P, ChainDesc* d, size_t* lds_out) {
    const int NT = N / 16;
    const int G = K / 128;
    const int units = NT < P ? NT : P;
    const int tmax = (NT + units - 1) / units;
    int kw = 1;
    for (int k : {8, 4, 2})
        if (tmax * k <= CH_NWAVE && G % k == 0) { kw = k; break; }
    for (int nch = 1; nch <= G; ++nch) {
        if (G % nch) continue;
        const int Gc = G / nch;
        if (Gc % kw) continue;
        if (nch > 1 && tmax > CH_NWAVE / kw) return false;   // a wave may own one tile only
        const size_t lds = chain_lds(M, Gc, tmax, kw);
        if (lds > QG_CH_LDS_BUDGET) continue;
        d->N = N;
        d->K = K;
        d->units = units;
        d->kw = kw;
        d->u = chain_u(Gc / kw);
        d->nchunks = nch;
        *lds_out = lds;
        return true;
    }
    return false;
}

hipError_t launch_chain(const ChainDesc* plan, int count, int M, size_t lds, unsigned* ws,
                        hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&w4a16_chain_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, QG_CH_LDS_BUDGET);
        attr_set = true;
    }
    const int P = chain_grid();
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&w4a16_chain_kernel), CH_NWAVE * 64, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
    void* args[] = {(void*)&plan, (void*)&count, (void*)&M, (void*)&ws};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&w4a16_chain_kernel), dim3(P),
                                      dim3(CH_NWAVE * 64), args, (unsigned)lds, s);
}

}  // namespace qg
