// Host-side launchers of the gfx950 kernels (private to libqgemm).  Shapes and
// pointers are validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace qg {

// Workspace of the K-split GEMMs (qgemm_w4a16, qgemm_w8a8_fp8 / _int8): the
// first kCounterBytes hold the completion counters (one 32-bit word per output
// tile or column strip, at most kMaxCounters of them), which every call that
// uses them leaves at zero; the offset terms and fp32 / int32 partial sums of
// the call follow.  The counters sit at the same offset for every shape, so a
// workspace that was zero-filled once serves calls of any shape in any order.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(unsigned));

// Devices whose host state (CU count, scratch address) is cached.
constexpr int kMaxDevices = 64;

// Library-owned scratch of qgemm_w4a16_noalloc: one array per device, the
// size limit of the workspace that entry point can serve.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// Device address of the current device's copy of that array (looked up once
// per device), or nullptr if the lookup fails.
void* noalloc_scratch();

// Compute units of the current device (queried once per device).  The kernel
// plans, and with them the workspace sizes, depend on it: a size query and the
// call it is made for must run with the same device current.
int device_cu_count();

// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device, once per
// device (`done` is the kernel's own record of the devices already set up).
void allow_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done);

// W4A16 path (w4a16.hip)
void launch_pack_int4_g128(const uint16_t* w, int K, int N, uint32_t* packed,
                           uint16_t* scales, hipStream_t s);
void launch_pack_int4_g128_mse(const uint16_t* w, int K, int N, int n_alpha, uint32_t* packed,
                               uint16_t* scales, hipStream_t s);
void launch_dequant_int4_g128(const uint32_t* packed, const uint16_t* scales, int K,
                              int N, uint16_t* w_out, uint8_t* codes_out, hipStream_t s);
size_t w4a16_workspace_bytes(int M, int N, int K);
const char* w4a16_kernel_for(int M, int N, int K);
void launch_qgemm_w4a16(const uint16_t* a, const uint32_t* packed, const uint16_t* scales,
                        uint16_t* y, int M, int N, int K, void* ws, hipStream_t s);

// Expert-grouped W4A16 (w4a16.hip)
constexpr int kGroupedMaxExperts = 1024;
int w4a16_grouped_max_items(int E, int T);
int w4a16_grouped_rows_per_item(int E, int T);
int grouped_small_ct(int NT, int E, int T, int ct);   // column tiles per small grouped workgroup
bool grouped_two_waves(int wg_per_expert, int E, int T);   // two waves per small grouped workgroup
size_t w4a16_grouped_workspace_bytes(int E, int T, int K);
void launch_qgemm_w4a16_grouped(const uint16_t* a, const int* offsets, const uint32_t* wq,
                                const uint16_t* sc, uint16_t* y, int E, int T, int N, int K,
                                void* ws, hipStream_t s);

// W4A8-FP8 (w4a8.hip)
void launch_qgemm_w4a8_fp8(const uint8_t* qa, const float* sa, const uint32_t* wq,
                           const uint16_t* sc, uint16_t* y, int M, int N, int K, hipStream_t s);
void launch_qgemm_w4a8_fp8_grouped(const uint8_t* qa, const float* sa, const int* offsets,
                                   const uint32_t* wq, const uint16_t* sc, uint16_t* y, int E, int T,
                                   int N, int K, hipStream_t s);
// bf16 routed rows in: the quantization inside the grouped GEMM for small
// items, else quant_act_per_token into the workspace first
size_t w4a8_grouped_dyn_workspace_bytes(int E, int T, int N, int K);
const char* w4a8_grouped_dyn_kernel_for(int E, int T, int N, int K);
void launch_qgemm_w4a8_fp8_grouped_dyn(const uint16_t* a, const int* offsets, const uint32_t* wq,
                                       const uint16_t* sc, uint16_t* y, int E, int T, int N, int K, void* ws,
                                       hipStream_t s);

// W8A8-FP8 path (fp8.hip)
void launch_quant_act_per_token(const uint16_t* a, int M, int K, uint8_t* q, float* s,
                                hipStream_t st);
void launch_quant_weight_fp8(const uint16_t* w, int K, int N, uint8_t* q, float* s,
                             hipStream_t st);
void launch_quant_act_per_token_i8(const uint16_t* a, int M, int K, int8_t* q, float* s,
                                   hipStream_t st);
void launch_quant_weight_i8(const uint16_t* w, int K, int N, int8_t* q, float* s, hipStream_t st);
void launch_qgemm_w8a8_i8(const int8_t* a, const float* sa, const int8_t* w, const float* sw,
                          uint16_t* y, int M, int N, int K, void* ws, hipStream_t st);
size_t w8a8_workspace_bytes(int M, int N, int K);   // both 8-bit formats
const char* w8a8_kernel_for(int M, int N, int K);
void launch_qgemm_w8a8_fp8(const uint8_t* a, const float* sa, const uint8_t* w,
                           const float* sw, uint16_t* y, int M, int N, int K, void* ws,
                           hipStream_t st);
// bf16 activations in: per-token quantization fused into the small-M GEMM, or
// quant_act into the workspace followed by the GEMM (both formats)
size_t w8a8_dyn_workspace_bytes(int M, int N, int K);
const char* w8a8_dyn_kernel_for(int M, int N, int K);
void launch_qgemm_w8a8_fp8_dyn(const uint16_t* a, const uint8_t* w, const float* sw, uint16_t* y,
                               int M, int N, int K, void* ws, hipStream_t st);
void launch_qgemm_w8a8_i8_dyn(const uint16_t* a, const int8_t* w, const float* sw, uint16_t* y,
                              int M, int N, int K, void* ws, hipStream_t st);

}  // namespace qg
