// Exercises every entry point of include/qgemm.h through abi.cpp with stub
// launchers (test infrastructure, host only): invalid arguments must return
// their status without launching; valid ones must reach exactly one launcher
// (the stub) and report QG_OK or, with no GPU present, QG_ERR_HIP.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer; prints "abi driver ok".
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/qgemm.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

// a valid call reaches one launcher; the status is OK, or HIP without a GPU
#define EXPECT_LAUNCH(call)                                                 \
    do {                                                                    \
        const int before = g_launches;                                      \
        const qg_status st = (call);                                        \
        EXPECT(st == QG_OK || st == QG_ERR_HIP);                            \
        EXPECT(g_launches > before);                                        \
    } while (0)

#define EXPECT_STATUS(call, want)                                           \
    do {                                                                    \
        const int before = g_launches;                                      \
        EXPECT((call) == (want));                                           \
        EXPECT(g_launches == before);                                       \
    } while (0)

int main() {
    // host buffers stand in for device memory: the stubs never dereference them
    std::vector<unsigned char> buf(1 << 22);
    unsigned char* base = buf.data();
    while (reinterpret_cast<uintptr_t>(base) % 256) ++base;
    auto* a16 = reinterpret_cast<uint16_t*>(base);
    auto* w32 = reinterpret_cast<uint32_t*>(base + 65536);
    auto* s16 = reinterpret_cast<uint16_t*>(base + 131072);
    auto* y16 = reinterpret_cast<uint16_t*>(base + 196608);
    auto* f32 = reinterpret_cast<float*>(base + 262144);
    auto* u8 = base + 327680;
    auto* i8 = reinterpret_cast<int8_t*>(base + 393216);
    auto* i32 = reinterpret_cast<int32_t*>(base + 458752);
    void* ws = base + 524288;

    // packing and dequantization
    EXPECT_LAUNCH(pack_int4_g128(a16, 256, 32, w32, s16, nullptr));
    EXPECT_STATUS(pack_int4_g128(nullptr, 256, 32, w32, s16, nullptr), QG_ERR_NULL);
    EXPECT_STATUS(pack_int4_g128(a16, 200, 32, w32, s16, nullptr), QG_ERR_SHAPE);
    EXPECT_STATUS(pack_int4_g128(a16 + 1, 256, 32, w32, s16, nullptr), QG_ERR_ALIGN);
    EXPECT_LAUNCH(pack_int4_g128_mse(a16, 256, 32, 100, w32, s16, nullptr));
    EXPECT_STATUS(pack_int4_g128_mse(a16, 256, 32, 0, w32, s16, nullptr), QG_ERR_SHAPE);
    EXPECT_LAUNCH(dequant_int4_g128(w32, s16, 256, 32, y16, u8, nullptr));
    EXPECT_STATUS(dequant_int4_g128(w32, s16, 256, 32, y16, u8 + 1, nullptr), QG_ERR_ALIGN);

    // W4A16
    EXPECT_LAUNCH(qgemm_w4a16(a16, w32, s16, y16, 4, 32, 256, nullptr, 0, nullptr));
    EXPECT_STATUS(qgemm_w4a16(a16, w32, s16, y16, 0, 32, 256, nullptr, 0, nullptr), QG_OK);
    EXPECT_STATUS(qgemm_w4a16(a16, w32, s16, y16, 4, 30, 256, nullptr, 0, nullptr), QG_ERR_SHAPE);
    EXPECT_STATUS(qgemm_w4a16(a16, w32, s16, y16, 100, 32, 256, nullptr, 0, nullptr), QG_ERR_NULL);
    EXPECT_STATUS(qgemm_w4a16(a16, w32, s16, y16, 100, 32, 256, ws, 100, nullptr), QG_ERR_WORKSPACE);
    EXPECT_LAUNCH(qgemm_w4a16(a16, w32, s16, y16, 100, 32, 256, ws, 4096, nullptr));
    EXPECT(qg_w4a16_workspace_bytes(100, 32, 256) == 4096);
    EXPECT(qg_w4a16_workspace_bytes(100, 30, 256) == 0);
    // allocation-free variant: the library's scratch serves the workspace
    EXPECT_LAUNCH(qgemm_w4a16_noalloc(a16, w32, s16, y16, 4, 32, 256, nullptr));
    EXPECT_LAUNCH(qgemm_w4a16_noalloc(a16, w32, s16, y16, 100, 32, 256, nullptr));
    EXPECT_STATUS(qgemm_w4a16_noalloc(a16, w32, s16, y16, 0, 32, 256, nullptr), QG_OK);
    EXPECT_STATUS(qgemm_w4a16_noalloc(nullptr, w32, s16, y16, 4, 32, 256, nullptr), QG_ERR_NULL);
    EXPECT_STATUS(qgemm_w4a16_noalloc(a16, w32, s16, y16, 4, 30, 256, nullptr), QG_ERR_SHAPE);
    EXPECT_STATUS(qgemm_w4a16_noalloc(a16 + 1, w32, s16, y16, 4, 32, 256, nullptr), QG_ERR_ALIGN);
    // a shape whose workspace exceeds the scratch (the stub's size query says 64 MiB)
    EXPECT_STATUS(qgemm_w4a16_noalloc(a16, w32, s16, y16, 100, 128000, 256, nullptr), QG_ERR_WORKSPACE);

    // grouped W4A16 and W4A8: few rows per expert need no workspace (NULL is
    // fine), many rows per expert (the large path) need one
    const int32_t off_ok[4] = {0, 3, 3, 8};
    for (int i = 0; i < 4; ++i) i32[i] = off_ok[i];
    EXPECT(qg_w4a16_grouped_workspace_bytes(3, 8, 32, 256) == 0);
    EXPECT_LAUNCH(qgemm_w4a16_grouped(a16, i32, w32, s16, y16, 3, 8, 32, 256, nullptr, 0, nullptr));
    EXPECT_STATUS(qgemm_w4a16_grouped(a16, i32, w32, s16, y16, 0, 8, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_SHAPE);
    const size_t gneed = qg_w4a16_grouped_workspace_bytes(3, 200, 32, 256);
    EXPECT(gneed > 0);
    EXPECT_LAUNCH(qgemm_w4a16_grouped(a16, i32, w32, s16, y16, 3, 200, 32, 256, ws, gneed, nullptr));
    EXPECT_STATUS(qgemm_w4a16_grouped(a16, i32, w32, s16, y16, 3, 200, 32, 256, ws, gneed - 4, nullptr),
                  QG_ERR_WORKSPACE);
    EXPECT_STATUS(qgemm_w4a16_grouped(a16, i32, w32, s16, y16, 3, 200, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_NULL);
    EXPECT_LAUNCH(qgemm_w4a8_fp8(u8, f32, w32, s16, y16, 40, 32, 256, nullptr));
    EXPECT_STATUS(qgemm_w4a8_fp8(u8, nullptr, w32, s16, y16, 40, 32, 256, nullptr), QG_ERR_NULL);
    EXPECT_LAUNCH(qgemm_w4a8_fp8_grouped(u8, f32, i32, w32, s16, y16, 3, 8, 32, 256, nullptr, 0, nullptr));
    EXPECT_LAUNCH(qgemm_w4a8_fp8_grouped(u8, f32, i32, w32, s16, y16, 3, 200, 32, 256, nullptr, 0, nullptr));
    const auto* off_odd = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(i32) + 2);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped(u8, f32, off_odd, w32, s16, y16, 3, 8, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_ALIGN);

    // grouped W4A8 on bf16 rows (quantization inside the call): none when fused,
    // the codes and scales otherwise
    EXPECT(qg_w4a8_grouped_dynamic_workspace_bytes(3, 8, 32, 256) == 0);
    EXPECT_LAUNCH(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 8, 32, 256, nullptr, 0, nullptr));
    const size_t gdneed = qg_w4a8_grouped_dynamic_workspace_bytes(3, 40, 32, 256);
    EXPECT(gdneed >= 40 * 256);
    EXPECT_LAUNCH(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 40, 32, 256, ws, gdneed, nullptr));
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 40, 32, 256, ws, gdneed - 1, nullptr),
                  QG_ERR_WORKSPACE);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 40, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_NULL);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 40, 32, 256,
                                                 reinterpret_cast<char*>(ws) + 4, gdneed, nullptr),
                  QG_ERR_ALIGN);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16 + 1, i32, w32, s16, y16, 3, 8, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_ALIGN);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 0, 8, 32, 256, nullptr, 0, nullptr),
                  QG_ERR_SHAPE);
    EXPECT_STATUS(qgemm_w4a8_fp8_grouped_dynamic(a16, i32, w32, s16, y16, 3, 0, 32, 256, nullptr, 0, nullptr),
                  QG_OK);

    // W8A8-FP8 and INT8
    EXPECT_LAUNCH(quant_act_per_token(a16, 4, 256, u8, f32, nullptr));
    EXPECT_STATUS(quant_act_per_token(a16, 4, 250, u8, f32, nullptr), QG_ERR_SHAPE);
    EXPECT_LAUNCH(quant_weight_fp8_per_channel(a16, 256, 32, u8, f32, nullptr));
    EXPECT_LAUNCH(qgemm_w8a8_fp8(u8, f32, u8, f32, y16, 4, 32, 256, nullptr, 0, nullptr));
    EXPECT_STATUS(qgemm_w8a8_fp8(u8, f32, u8, f32, y16, 100, 32, 256, nullptr, 0, nullptr), QG_ERR_NULL);
    EXPECT_LAUNCH(qgemm_w8a8_fp8(u8, f32, u8, f32, y16, 100, 32, 256, ws, 2048, nullptr));
    EXPECT_LAUNCH(quant_act_per_token_int8(a16, 4, 256, i8, f32, nullptr));
    EXPECT_LAUNCH(quant_weight_int8_per_channel(a16, 256, 32, i8, f32, nullptr));
    EXPECT_LAUNCH(qgemm_w8a8_int8(i8, f32, i8, f32, y16, 4, 32, 256, nullptr, 0, nullptr));
    EXPECT_STATUS(qgemm_w8a8_int8(i8, f32, i8, f32, y16, 4, 32, 131072 + 128, nullptr, 0, nullptr),
                  QG_ERR_SHAPE);

    // W8A8 with the activation quantization inside the call (bf16 activations)
    EXPECT_LAUNCH(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 4, 32, 256, nullptr, 0, nullptr));
    EXPECT_LAUNCH(qgemm_w8a8_int8_dynamic(a16, i8, f32, y16, 4, 32, 256, nullptr, 0, nullptr));
    const size_t dneed = qg_w8a8_dynamic_workspace_bytes(40, 32, 256);
    EXPECT(dneed >= (size_t)40 * 256);
    EXPECT_LAUNCH(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 40, 32, 256, ws, dneed, nullptr));
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 40, 32, 256, ws, dneed - 1, nullptr),
                  QG_ERR_WORKSPACE);
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 40, 32, 256, nullptr, 0, nullptr), QG_ERR_NULL);
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(nullptr, u8, f32, y16, 4, 32, 256, nullptr, 0, nullptr), QG_ERR_NULL);
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(a16 + 1, u8, f32, y16, 4, 32, 256, nullptr, 0, nullptr), QG_ERR_ALIGN);
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 4, 30, 256, nullptr, 0, nullptr), QG_ERR_SHAPE);
    EXPECT_STATUS(qgemm_w8a8_fp8_dynamic(a16, u8, f32, y16, 0, 32, 256, nullptr, 0, nullptr), QG_OK);
    EXPECT_STATUS(qgemm_w8a8_int8_dynamic(a16, i8, f32, y16, 4, 32, 131072 + 128, nullptr, 0, nullptr),
                  QG_ERR_SHAPE);

    // strings
    EXPECT(qg_status_string(QG_OK) != nullptr && qg_status_string(1234) != nullptr);
    EXPECT(qg_version() != nullptr);

    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("abi driver ok (%d stub launches)\n", g_launches);
    return 0;
}
