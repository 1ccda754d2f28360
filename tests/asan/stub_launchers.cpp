// Host-only stand-ins for the gfx950 launchers of libqgemm (test
// infrastructure): they record each call and touch no memory, so that the
// C-ABI layer (abi.cpp) can be built and exercised under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  Size queries return
// simple fixed formulas; the driver only relies on their being consistent
// with what abi.cpp checks.
#include <hip/hip_runtime.h>

#include "launch.h"

int g_launches = 0;

namespace qg {

void launch_pack_int4_g128(const uint16_t*, int, int, uint32_t*, uint16_t*, hipStream_t) { ++g_launches; }
void launch_pack_int4_g128_mse(const uint16_t*, int, int, int, uint32_t*, uint16_t*, hipStream_t) { ++g_launches; }
void launch_dequant_int4_g128(const uint32_t*, const uint16_t*, int, int, uint16_t*, uint8_t*, hipStream_t) { ++g_launches; }
size_t w4a16_workspace_bytes(int M, int N, int) { return M > 64 ? (N > 100000 ? (size_t(64) << 20) : 4096) : 0; }
static unsigned char g_scratch[256];
void* noalloc_scratch() { return g_scratch; }
const char* w4a16_kernel_for(int, int, int) { return "stub"; }
void launch_qgemm_w4a16(const uint16_t*, const uint32_t*, const uint16_t*, uint16_t*, int, int, int, void*,
                        hipStream_t) { ++g_launches; }
int w4a16_grouped_max_items(int E, int T) { return (T < E ? T : E) + (T + 15) / 16; }
int w4a16_grouped_rows_per_item(int, int) { return 16; }
// grouped: a workspace (the large path's offset terms) from a mean of 33 rows per expert
size_t w4a16_grouped_workspace_bytes(int E, int T, int K) {
    const int active = T < E ? T : E;
    return active > 0 && T >= 33 * active ? (size_t)(K / 128) * (T + 128) * sizeof(float) : 0;
}
void launch_qgemm_w4a16_grouped(const uint16_t*, const int*, const uint32_t*, const uint16_t*, uint16_t*, int,
                                int, int, int, void*, hipStream_t) { ++g_launches; }
void launch_qgemm_w4a8_fp8(const uint8_t*, const float*, const uint32_t*, const uint16_t*, uint16_t*, int, int,
                           int, hipStream_t) { ++g_launches; }
void launch_qgemm_w4a8_fp8_grouped(const uint8_t*, const float*, const int*, const uint32_t*, const uint16_t*,
                                   uint16_t*, int, int, int, int, hipStream_t) { ++g_launches; }
// grouped W4A8 on bf16 rows: fused (no workspace) below 17 rows, else codes and scales
size_t w4a8_grouped_dyn_workspace_bytes(int, int T, int, int K) {
    return T > 16 ? (size_t)T * K + (size_t)T * 4 : 0;
}
const char* w4a8_grouped_dyn_kernel_for(int, int, int, int) { return "stub"; }
void launch_qgemm_w4a8_fp8_grouped_dyn(const uint16_t*, const int*, const uint32_t*, const uint16_t*, uint16_t*,
                                       int, int, int, int, void*, hipStream_t) { ++g_launches; }
void launch_quant_act_per_token(const uint16_t*, int, int, uint8_t*, float*, hipStream_t) { ++g_launches; }
void launch_quant_weight_fp8(const uint16_t*, int, int, uint8_t*, float*, hipStream_t) { ++g_launches; }
void launch_quant_act_per_token_i8(const uint16_t*, int, int, int8_t*, float*, hipStream_t) { ++g_launches; }
void launch_quant_weight_i8(const uint16_t*, int, int, int8_t*, float*, hipStream_t) { ++g_launches; }
void launch_qgemm_w8a8_i8(const int8_t*, const float*, const int8_t*, const float*, uint16_t*, int, int, int,
                          void*, hipStream_t) { ++g_launches; }
size_t w8a8_workspace_bytes(int M, int, int) { return M > 64 ? 2048 : 0; }
const char* w8a8_kernel_for(int, int, int) { return "stub"; }
void launch_qgemm_w8a8_fp8(const uint8_t*, const float*, const uint8_t*, const float*, uint16_t*, int, int,
                           int, void*, hipStream_t) { ++g_launches; }
// bf16-input W8A8: fused (no workspace) up to 16 rows, else codes in the workspace
size_t w8a8_dyn_workspace_bytes(int M, int N, int K) {
    return M <= 16 ? 0 : w8a8_workspace_bytes(M, N, K) + (size_t)M * K + (size_t)M * 4;
}
const char* w8a8_dyn_kernel_for(int, int, int) { return "stub"; }
void launch_qgemm_w8a8_fp8_dyn(const uint16_t*, const uint8_t*, const float*, uint16_t*, int, int, int, void*,
                               hipStream_t) { ++g_launches; }
void launch_qgemm_w8a8_i8_dyn(const uint16_t*, const int8_t*, const float*, uint16_t*, int, int, int, void*,
                              hipStream_t) { ++g_launches; }

}  // namespace qg
