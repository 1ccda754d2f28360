// Device-side helpers shared by the gfx950 kernels of libqgemm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace qg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 --------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

// IEEE round-to-nearest-even fp32 -> bf16 bit pattern; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- INT4 unpack ------------------------------------------------------------
// A native word holds eight 4-bit codes; nibble slots j and j+4 hold the rows
// 2j and 2j+1 of the word's 8-row slice.  Masking both nibbles into the low
// mantissa bits of the bf16 pattern 0x4300 (= 128.0) makes the exact bf16 pair
// (128 + code[2j], 128 + code[2j+1]): one shift and one AND-OR per two weights
// ("When quantization pays", section "Counting c": the same masks).
__device__ __forceinline__ uint32_t int4_pair_biased_bf16x2(uint32_t word, int j) {
    return ((word >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
}

// Eight weights of one word -> MFMA operand (rows 0..7 in order), values 128 + code.
__device__ __forceinline__ bf16x8 int4_word_biased_bf16x8(uint32_t word) {
    u32x4 v;
    v.x = int4_pair_biased_bf16x2(word, 0);
    v.y = int4_pair_biased_bf16x2(word, 1);
    v.z = int4_pair_biased_bf16x2(word, 2);
    v.w = int4_pair_biased_bf16x2(word, 3);
    return __builtin_bit_cast(bf16x8, v);
}

// The unpack constants live in VGPRs: a VOP3 instruction reads at most one
// scalar or literal operand here, and keeping both the nibble mask and the
// bf16 magic in vector registers lets every pair compile to one v_and_or_b32
// (3 shifts + 4 AND-ORs per 8 weights).
struct Int4Unpacker {
    uint32_t mask, magic;
    __device__ __forceinline__ Int4Unpacker() {
        asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(mask));
        asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(magic));
    }
    __device__ __forceinline__ bf16x8 operator()(uint32_t w) const {
        u32x4 v;
        v.x = (w & mask) | magic;
        v.y = ((w >> 4) & mask) | magic;
        v.z = ((w >> 8) & mask) | magic;
        v.w = ((w >> 12) & mask) | magic;
        return as_bf16x8(v);
    }
};

// ---- MFMA wrappers ------------------------------------------------------------
// 16x16x32 bf16, fp32 accumulate.  A: lane l holds row l%16, 8 consecutive k of
// the 32-wide step; B: lane l holds column l%16, the same 8 k.  D: lane l holds
// column l%16, rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16, fp32 accumulate.  A: lane l holds row l%32, k = 8*(l/32) .. +7;
// B: lane l holds column l%32, the same 8 k; D: register i of lane l holds
// row 8*(i/4) + 4*(l/32) + i%4, column l%32.  On gfx950 this form sustains about
// twice the bf16 rate of the 16x16x32 form.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x128 OCP e4m3 x e4m3, fp32 accumulate (block scales fixed at 2^0).
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}


// 128-bit direct-to-LDS load: lane l's 16 bytes from src land at lds_base + 16 * l
// (lds_base must be the same in every lane of the wave).
__device__ __forceinline__ void load_lds_b128(const u32x4* src, u32x4* lds_base) {
    __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// ---- compile-time loops ----------------------------------------------------------
template <int V>
using ic = std::integral_constant<int, V>;

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(ic<I>{}), ...);
}
// f(ic<0>{}), f(ic<1>{}), ..., f(ic<N-1>{}) in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- buffer-resource loads ----------------------------------------------------------
// A raw buffer resource over [base, base + bytes).  A load whose offset lies at
// or past `bytes` returns zero and makes no memory access, so `bytes = 0` turns
// a request into a no-op without a branch (dword 3 is the gfx9-family format
// word for untyped buffer access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// 16 bytes at byte offset `off`, streaming (non-temporal) hint
__device__ __forceinline__ u32x4 buffer_load_b128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ uint32_t buffer_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// ---- register ring pipeline ------------------------------------------------------------
// n items through D register buffers: item i lives in buffer i % D and is
// requested D - 1 items before it is consumed.  load(slot) requests the next
// item in order (the caller keeps that cursor and issues an empty request past
// the last item, see make_rsrc), so every request is unconditional and the
// compiler's memory-counter waits stay exact; compute(slot) consumes the next
// item.  The scheduling barriers keep each request ahead of the compute that
// follows it.
template <int D, typename Load, typename Compute>
__device__ __forceinline__ void ring_pipeline(int n, Load&& load, Compute&& compute) {
    for (int it = 0; it < n; it += D) {
        static_for<D>([&](auto s) {
            load(ic<(decltype(s)::value + D - 1) % D>{});
            __builtin_amdgcn_sched_barrier(0);
            if (it + decltype(s)::value < n) compute(s);
        });
    }
}
// the first D - 1 requests of ring_pipeline, issued ahead of other work
template <int D, typename Load>
__device__ __forceinline__ void ring_prologue(Load&& load) {
    static_for<D - 1>([&](auto s) {
        load(s);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// The same copy issued as inline assembly: the compiler does not track it, so
// it adds no waits of its own between copies and later LDS accesses (it cannot
// tell LDS stages apart and would wait for every copy).  The caller waits for
// the copy with s_waitcnt vmcnt and publishes it with a barrier.  The LDS
// address goes in through M0 as an input operand, so the compiler itself sets
// the register and knows its value afterwards.
__device__ __forceinline__ void lds_copy_b128(const void* src, const void* lds_dst) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_dst;
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// ---- cross-workgroup handoff ----------------------------------------------------
// A workgroup has written its partial results with agent-scope atomic stores
// (written through to the memory side, where every XCD reads them) and now
// counts its arrival; the workgroup whose increment completes the count reads
// every slot.  Ordering: each wave first waits until all of its own stores have
// completed (a workgroup barrier alone orders LDS traffic only, not the other
// waves' outstanding global stores), the barrier then ensures every wave got
// there, and only then does one thread increment the counter.  So every slot
// store of this workgroup is complete before its increment is visible, and the
// last arriver, which issues its agent-scope slot loads only after its own
// increment has returned, reads each slot after it was written.  Returns true
// in every thread of the last-arriving workgroup.
__device__ __forceinline__ bool arrive_and_check_last(unsigned* counter, unsigned arrivals,
                                                      int* flag_lds) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        *flag_lds = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    arrivals - 1u;
    __syncthreads();
    return *flag_lds != 0;
}

__device__ __forceinline__ i32x8 cat_i32x8(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).  This
// remaps workgroup id so that each XCD receives a contiguous run of tile ids,
// so tiles that are neighbours in the caller's order share that XCD's L2.
constexpr int NUM_XCD = 8;
__device__ __forceinline__ int xcd_tile(int id, int total) {
    const int per = total / NUM_XCD;
    return id < per * NUM_XCD ? (id % NUM_XCD) * per + id / NUM_XCD : id;
}

// Expert-grouped large tiles on a 1-D grid of NX column tiles x items (items
// rounded up to a multiple of NUM_XCD): workgroup L takes column tile x and
// item y such that every column tile of an item runs on one XCD (the one
// workgroup L % NUM_XCD is dealt to), so the item's activation rows are
// fetched into one L2 and read by its NX workgroups from there.
__device__ __forceinline__ void grouped_xcd_item(int L, int NX, int& x, int& y) {
    const int q = L / NUM_XCD;
    x = q % NX;
    y = (q / NX) * NUM_XCD + L % NUM_XCD;
}

// Column tile x and item y of an expert-grouped workgroup: on a 1-D grid of
// NX x (items rounded up to NUM_XCD) workgroups through grouped_xcd_item
// (xcd != 0), else on the 2-D grid (NX, items).
__device__ __forceinline__ void grouped_xy(int xcd, int NX, int& x, int& y) {
    if (xcd) {
        grouped_xcd_item(blockIdx.x, NX, x, y);
    } else {
        x = blockIdx.x;
        y = blockIdx.y;
    }
}

// whether the 1-D grid of grouped_xy fits a dispatch (fewer than 2^32 work-items)
inline int grouped_xcd_fits(int NX, int items, int threads) {
    const unsigned long long wg = (unsigned long long)NX * ((items + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
    return wg * (unsigned long long)threads < (1ull << 32) ? 1 : 0;
}

// the grid of grouped_xy
inline dim3 grouped_grid(int xcd, int NX, int items) {
    return xcd ? dim3((unsigned)(NX * ((items + NUM_XCD - 1) / NUM_XCD * NUM_XCD))) : dim3(NX, items);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---- expert-grouped work items ----------------------------------------------
// An expert-grouped call (E experts, T routed rows, expert e owning rows
// offsets[e] .. offsets[e+1] - 1) is cut into work items of at most R rows:
// each expert's rows in chunks of R, the items numbered in expert order and in
// row order within an expert.  Offsets are clamped into [0, T] with
// r0 <= r1 per expert, so malformed offsets stay in bounds.  The GEMM grid
// holds one workgroup row per item up to the bound min(E, T) + ceil(T / R),
// which well-formed offsets never exceed; items past it are dropped.
//
// Every wave finds the item `it` of its workgroup on its own, with no launch
// and no memory round trip before the GEMM: the experts are taken 64 at a
// time, expert 64 j + lane on lane `lane` (one coalesced pair of offset loads
// per block, the next block's in flight while this one is counted); a wave
// prefix sum of the blocks' chunk counts numbers the items, and the block and
// lane holding item `it` supply (expert, first row, rows), read into scalar
// registers.  All waves of a workgroup reach the same answer (measured:
// cheaper than one wave deriving it and handing it over through LDS behind a
// barrier).  false: fewer than it + 1 items (nothing to do).
constexpr int GROUPED_MAX_E = 1024;

struct GroupedItem {
    int e, r0, rows;
};

template <int R>
__device__ __forceinline__ bool grouped_item(const int* __restrict__ offsets, int E, int T, int it,
                                             GroupedItem& item) {
    const int lane = threadIdx.x & 63;
    const int nblk = (E + 63) >> 6;
    int a = offsets[min(lane, E)];
    int b = offsets[min(lane + 1, E)];
    int carry = 0;                                   // items of the blocks before
    for (int j = 0; j < nblk; ++j) {
        const int e = 64 * j + lane;
        int na = 0, nb = 0;
        if (j + 1 < nblk) {
            na = offsets[min(e + 64, E)];
            nb = offsets[min(e + 65, E)];
        }
        const int lo = e < E ? min(max(a, 0), T) : 0;
        const int hi = e < E ? min(max(b, lo), T) : 0;
        const int c = (hi - lo + R - 1) / R;
        int incl = c;                                // inclusive prefix over the lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        incl += carry;
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (it < total) {                            // uniform; carry <= it, so one lane owns it
            const int first = incl - c;
            const int src = __builtin_ctzll(__ballot(it >= first && it < incl));
            const int r0 = lo + (it - first) * R;
            item.e = __builtin_amdgcn_readlane(e, src);
            item.r0 = __builtin_amdgcn_readlane(r0, src);
            item.rows = __builtin_amdgcn_readlane(min(R, hi - r0), src);
            return true;
        }
        carry = total;
        a = na;
        b = nb;
    }
    return false;
}

// Offset terms of a staged activation slice: corr[g * 16 + m] = -136 * (sum of
// row m's 128 activations of group g).  Above 8 rows on the MFMA: the staged
// fragments (arow: this lane's row min(col, M-1), k-quarter kq) times a B
// operand of bf16 -136 (exact products) give every column the same row sums,
// and lane (col 0, kq) of the result holds rows 4kq .. 4kq+3.  Up to 8 rows a
// thread per (group, row) adds the 128 values in order (measured: cheaper than
// the MFMA pass when few rows need it).
__device__ __forceinline__ void decode_offset_terms(const unsigned char* lds, int rowb, float* corr,
                                                    const unsigned char* arow, int M, int G, int tid,
                                                    int wave, int col, int kq, int nwave) {
    if (M > 8) {
        const bf16x8 neg136 = as_bf16x8(u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
        for (int g = wave; g < G; g += nwave) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc = mfma_bf16_16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(arow + g * 256 + t * 64)),
                                         neg136, acc);
            if (col == 0) *reinterpret_cast<f32x4*>(corr + g * 16 + 4 * kq) = acc;
        }
        return;
    }
    for (int p = tid; p < G * M; p += nwave * 64) {
        const int g = p / M;
        const int m = p - g * M;
        const u32x4* row = reinterpret_cast<const u32x4*>(lds + (size_t)m * rowb + g * 256);
        float sum = 0.0f;
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
            const u32x4 v = row[i];
            sum += bf16_to_f32(v.x & 0xffffu) + bf16_to_f32(v.x >> 16);
            sum += bf16_to_f32(v.y & 0xffffu) + bf16_to_f32(v.y >> 16);
            sum += bf16_to_f32(v.z & 0xffffu) + bf16_to_f32(v.z >> 16);
            sum += bf16_to_f32(v.w & 0xffffu) + bf16_to_f32(v.w >> 16);
        }
        corr[g * 16 + m] = -136.0f * sum;
    }
}

}  // namespace qg
