// C ABI of libqgemm (declared in include/qgemm.h): argument validation on the
// host, before anything is launched, then dispatch to the gfx950 launchers.
#include <hip/hip_runtime.h>

#include "../../include/qgemm.h"
#include "launch.h"

namespace {

// Limits that keep every index the kernels form inside its integer type.
constexpr int64_t kMaxDim = int64_t(1) << 24;        // M, N
constexpr int64_t kMaxK = int64_t(1) << 20;          // K
constexpr int64_t kMaxElems = int64_t(1) << 38;      // elements of one matrix
constexpr int64_t kMaxKInt8 = int64_t(1) << 17;      // int8 GEMM: 127^2 * K fits int32

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// K % 128, N % 16, bounds.  M may be 0.
bool shape_ok(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0) return false;
    if (K % 128 != 0 || N % 16 != 0) return false;
    if (M > kMaxDim || N > kMaxDim || K > kMaxK) return false;
    if (N * K > kMaxElems || M * K > kMaxElems || M * N > kMaxElems) return false;
    return true;
}

// Expert-grouped shapes: E experts of [K, N], T routed rows.
bool grouped_ok(int64_t E, int64_t T, int64_t N, int64_t K) {
    if (E < 1 || E > qg::kGroupedMaxExperts || !shape_ok(T, N, K)) return false;
    if (E * N * K > 64 * kMaxElems) return false;
    return T == 0 || qg::w4a16_grouped_max_items((int)E, (int)T) <= 65535;
}

qg_status launched() {
    return hipGetLastError() == hipSuccess ? QG_OK : QG_ERR_HIP;
}

hipStream_t as_stream(qg_stream s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* qg_status_string(int status) {
    switch (status) {
        case QG_OK: return "ok";
        case QG_ERR_NULL: return "a required pointer is NULL";
        case QG_ERR_SHAPE:
            return "invalid shape (need M >= 0, N > 0, K > 0, K % 128 == 0, N % 16 == 0, within "
                   "size limits)";
        case QG_ERR_ALIGN: return "a pointer is not aligned (matrices 16 bytes, vectors 4 bytes)";
        case QG_ERR_WORKSPACE: return "workspace smaller than the size query requires";
        case QG_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown status";
    }
}

const char* qg_version(void) { return "qgemm-gfx950 0.1.0"; }

size_t qg_int4_g128_packed_bytes(int64_t K, int64_t N) {
    if (!shape_ok(0, N, K)) return 0;
    return (size_t)(K * N / 2);
}

size_t qg_int4_g128_scale_bytes(int64_t K, int64_t N) {
    if (!shape_ok(0, N, K)) return 0;
    return (size_t)(K / 128 * N * 2);
}

const char* qg_w4a16_kernel_for(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return "";
    return qg::w4a16_kernel_for((int)M, (int)N, (int)K);
}

const char* qg_w8a8_kernel_for(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return "";
    return qg::w8a8_kernel_for((int)M, (int)N, (int)K);
}

size_t qg_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return 0;
    return qg::w4a16_workspace_bytes((int)M, (int)N, (int)K);
}

size_t qg_w4a16_grouped_workspace_bytes(int64_t E, int64_t T, int64_t N, int64_t K) {
    if (!grouped_ok(E, T, N, K)) return 0;
    return qg::w4a16_grouped_workspace_bytes((int)E, (int)T, (int)K);
}

size_t qg_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return 0;
    return qg::w8a8_workspace_bytes((int)M, (int)N, (int)K);
}

qg_status pack_int4_g128(const uint16_t* w_bf16, int K, int N, uint32_t* packed,
                         uint16_t* scales, qg_stream stream) {
    if (!w_bf16 || !packed || !scales) return QG_ERR_NULL;
    if (!shape_ok(0, N, K)) return QG_ERR_SHAPE;
    if (!aligned(w_bf16, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return QG_ERR_ALIGN;
    qg::launch_pack_int4_g128(w_bf16, K, N, packed, scales, as_stream(stream));
    return launched();
}

qg_status pack_int4_g128_mse(const uint16_t* w_bf16, int K, int N, int n_alpha, uint32_t* packed,
                             uint16_t* scales, qg_stream stream) {
    if (!w_bf16 || !packed || !scales) return QG_ERR_NULL;
    if (!shape_ok(0, N, K) || n_alpha < 1 || n_alpha > 65535) return QG_ERR_SHAPE;
    if (!aligned(w_bf16, 16) || !aligned(packed, 16) || !aligned(scales, 4)) return QG_ERR_ALIGN;
    qg::launch_pack_int4_g128_mse(w_bf16, K, N, n_alpha, packed, scales, as_stream(stream));
    return launched();
}

qg_status dequant_int4_g128(const uint32_t* packed, const uint16_t* scales, int K, int N,
                            uint16_t* w_bf16_out, uint8_t* codes_out, qg_stream stream) {
    if (!packed || !scales || !w_bf16_out) return QG_ERR_NULL;
    if (!shape_ok(0, N, K)) return QG_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(w_bf16_out, 16) ||
        (codes_out && !aligned(codes_out, 16)))
        return QG_ERR_ALIGN;
    qg::launch_dequant_int4_g128(packed, scales, K, N, w_bf16_out, codes_out, as_stream(stream));
    return launched();
}

qg_status qgemm_w4a16(const uint16_t* a_bf16, const uint32_t* packed, const uint16_t* scales,
                      uint16_t* y_bf16, int M, int N, int K, void* workspace,
                      size_t workspace_bytes, qg_stream stream) {
    if (!shape_ok(M, N, K)) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_bf16 || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w4a16_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
    }
    qg::launch_qgemm_w4a16(a_bf16, packed, scales, y_bf16, M, N, K, workspace, as_stream(stream));
    return launched();
}

qg_status qgemm_w4a16_noalloc(const uint16_t* a_bf16, const uint32_t* packed, const uint16_t* scales,
                              uint16_t* y_bf16, int M, int N, int K, qg_stream stream) {
    static_assert(qg::kNoAllocScratchBytes == QG_NOALLOC_SCRATCH_BYTES, "scratch limit of the header");
    if (!shape_ok(M, N, K)) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_bf16 || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(packed, 16) || !aligned(scales, 4) || !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w4a16_workspace_bytes(M, N, K);
    if (need > qg::kNoAllocScratchBytes) return QG_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0 && (ws = qg::noalloc_scratch()) == nullptr) return QG_ERR_HIP;
    qg::launch_qgemm_w4a16(a_bf16, packed, scales, y_bf16, M, N, K, ws, as_stream(stream));
    return launched();
}

qg_status qgemm_w4a16_grouped(const uint16_t* a_bf16, const int32_t* offsets,
                              const uint32_t* packed, const uint16_t* scales, uint16_t* y_bf16,
                              int E, int T, int N, int K, void* workspace, size_t workspace_bytes,
                              qg_stream stream) {
    if (!grouped_ok(E, T, N, K)) return QG_ERR_SHAPE;
    if (T == 0) return QG_OK;
    if (!a_bf16 || !offsets || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(offsets, 4) || !aligned(packed, 16) ||
        !aligned(scales, 4) || !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w4a16_grouped_workspace_bytes(E, T, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return QG_ERR_ALIGN;
    }
    qg::launch_qgemm_w4a16_grouped(a_bf16, offsets, packed, scales, y_bf16, E, T, N, K, workspace,
                                   as_stream(stream));
    return launched();
}

qg_status quant_act_per_token(const uint16_t* a_bf16, int M, int K, uint8_t* a_e4m3,
                              float* a_scale, qg_stream stream) {
    if (M < 0 || K <= 0 || K % 8 != 0 || M > kMaxDim || K > kMaxK) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_bf16 || !a_e4m3 || !a_scale) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(a_e4m3, 16) || !aligned(a_scale, 4)) return QG_ERR_ALIGN;
    qg::launch_quant_act_per_token(a_bf16, M, K, a_e4m3, a_scale, as_stream(stream));
    return launched();
}

qg_status quant_weight_fp8_per_channel(const uint16_t* w_bf16, int K, int N, uint8_t* w_e4m3,
                                       float* w_scale, qg_stream stream) {
    if (!w_bf16 || !w_e4m3 || !w_scale) return QG_ERR_NULL;
    if (!shape_ok(0, N, K)) return QG_ERR_SHAPE;
    if (!aligned(w_bf16, 16) || !aligned(w_e4m3, 16) || !aligned(w_scale, 4)) return QG_ERR_ALIGN;
    qg::launch_quant_weight_fp8(w_bf16, K, N, w_e4m3, w_scale, as_stream(stream));
    return launched();
}

qg_status qgemm_w8a8_fp8(const uint8_t* a_e4m3, const float* a_scale, const uint8_t* w_e4m3,
                         const float* w_scale, uint16_t* y_bf16, int M, int N, int K,
                         void* workspace, size_t workspace_bytes, qg_stream stream) {
    if (!shape_ok(M, N, K)) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_e4m3 || !a_scale || !w_e4m3 || !w_scale || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_e4m3, 16) || !aligned(a_scale, 4) || !aligned(w_e4m3, 16) ||
        !aligned(w_scale, 4) || !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w8a8_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
    }
    qg::launch_qgemm_w8a8_fp8(a_e4m3, a_scale, w_e4m3, w_scale, y_bf16, M, N, K, workspace,
                              as_stream(stream));
    return launched();
}

// ---- W4A8-FP8: INT4 g128 weights x per-token e4m3 activations ----

qg_status qgemm_w4a8_fp8(const uint8_t* a_e4m3, const float* a_scale, const uint32_t* packed,
                         const uint16_t* scales, uint16_t* y_bf16, int M, int N, int K,
                         qg_stream stream) {
    if (!shape_ok(M, N, K) || (M + 63) / 64 > 65535) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_e4m3 || !a_scale || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_e4m3, 16) || !aligned(a_scale, 4) || !aligned(packed, 16) || !aligned(scales, 4) ||
        !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    qg::launch_qgemm_w4a8_fp8(a_e4m3, a_scale, packed, scales, y_bf16, M, N, K, as_stream(stream));
    return launched();
}

qg_status qgemm_w4a8_fp8_grouped(const uint8_t* a_e4m3, const float* a_scale, const int32_t* offsets,
                                 const uint32_t* packed, const uint16_t* scales, uint16_t* y_bf16,
                                 int E, int T, int N, int K, void* /*workspace*/, size_t /*workspace_bytes*/,
                                 qg_stream stream) {
    if (!grouped_ok(E, T, N, K)) return QG_ERR_SHAPE;
    if (T == 0) return QG_OK;
    if (!a_e4m3 || !a_scale || !offsets || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_e4m3, 16) || !aligned(a_scale, 4) || !aligned(offsets, 4) || !aligned(packed, 16) ||
        !aligned(scales, 4) || !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    qg::launch_qgemm_w4a8_fp8_grouped(a_e4m3, a_scale, offsets, packed, scales, y_bf16, E, T, N, K,
                                      as_stream(stream));
    return launched();
}

size_t qg_w4a8_grouped_dynamic_workspace_bytes(int64_t E, int64_t T, int64_t N, int64_t K) {
    if (!grouped_ok(E, T, N, K)) return 0;
    return qg::w4a8_grouped_dyn_workspace_bytes((int)E, (int)T, (int)N, (int)K);
}

const char* qg_w4a8_grouped_dynamic_kernel_for(int64_t E, int64_t T, int64_t N, int64_t K) {
    if (!grouped_ok(E, T, N, K)) return "";
    return qg::w4a8_grouped_dyn_kernel_for((int)E, (int)T, (int)N, (int)K);
}

qg_status qgemm_w4a8_fp8_grouped_dynamic(const uint16_t* a_bf16, const int32_t* offsets, const uint32_t* packed,
                                         const uint16_t* scales, uint16_t* y_bf16, int E, int T, int N, int K,
                                         void* workspace, size_t workspace_bytes, qg_stream stream) {
    if (!grouped_ok(E, T, N, K)) return QG_ERR_SHAPE;
    if (T == 0) return QG_OK;
    if (!a_bf16 || !offsets || !packed || !scales || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(offsets, 4) || !aligned(packed, 16) || !aligned(scales, 4) ||
        !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w4a8_grouped_dyn_workspace_bytes(E, T, N, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
    }
    qg::launch_qgemm_w4a8_fp8_grouped_dyn(a_bf16, offsets, packed, scales, y_bf16, E, T, N, K, workspace,
                                          as_stream(stream));
    return launched();
}

// ---- W8A8-INT8: the same kernels with int8 codes and int32 accumulation ----

size_t qg_w8a8_int8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K) || K > kMaxKInt8) return 0;
    return qg::w8a8_workspace_bytes((int)M, (int)N, (int)K);
}

qg_status quant_act_per_token_int8(const uint16_t* a_bf16, int M, int K, int8_t* a_i8,
                                   float* a_scale, qg_stream stream) {
    if (M < 0 || K <= 0 || K % 8 != 0 || M > kMaxDim || K > kMaxK) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_bf16 || !a_i8 || !a_scale) return QG_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(a_i8, 16) || !aligned(a_scale, 4)) return QG_ERR_ALIGN;
    qg::launch_quant_act_per_token_i8(a_bf16, M, K, a_i8, a_scale, as_stream(stream));
    return launched();
}

qg_status quant_weight_int8_per_channel(const uint16_t* w_bf16, int K, int N, int8_t* w_i8,
                                        float* w_scale, qg_stream stream) {
    if (!w_bf16 || !w_i8 || !w_scale) return QG_ERR_NULL;
    if (!shape_ok(0, N, K)) return QG_ERR_SHAPE;
    if (!aligned(w_bf16, 16) || !aligned(w_i8, 16) || !aligned(w_scale, 4)) return QG_ERR_ALIGN;
    qg::launch_quant_weight_i8(w_bf16, K, N, w_i8, w_scale, as_stream(stream));
    return launched();
}

qg_status qgemm_w8a8_int8(const int8_t* a_i8, const float* a_scale, const int8_t* w_i8,
                          const float* w_scale, uint16_t* y_bf16, int M, int N, int K,
                          void* workspace, size_t workspace_bytes, qg_stream stream) {
    if (!shape_ok(M, N, K) || K > kMaxKInt8) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    if (!a_i8 || !a_scale || !w_i8 || !w_scale || !y_bf16) return QG_ERR_NULL;
    if (!aligned(a_i8, 16) || !aligned(a_scale, 4) || !aligned(w_i8, 16) || !aligned(w_scale, 4) ||
        !aligned(y_bf16, 16))
        return QG_ERR_ALIGN;
    const size_t need = qg::w8a8_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
    }
    qg::launch_qgemm_w8a8_i8(a_i8, a_scale, w_i8, w_scale, y_bf16, M, N, K, workspace,
                             as_stream(stream));
    return launched();
}

size_t qg_w8a8_dynamic_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return 0;
    return qg::w8a8_dyn_workspace_bytes((int)M, (int)N, (int)K);
}

const char* qg_w8a8_dynamic_kernel_for(int64_t M, int64_t N, int64_t K) {
    if (!shape_ok(M, N, K)) return "";
    return qg::w8a8_dyn_kernel_for((int)M, (int)N, (int)K);
}

// Shared checks of the two bf16-input W8A8 entry points.
static qg_status dynamic_args_ok(const uint16_t* a, const void* w, const float* sw, const uint16_t* y, int M,
                                 int N, int K, void* workspace, size_t workspace_bytes) {
    if (!a || !w || !sw || !y) return QG_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(sw, 4) || !aligned(y, 16)) return QG_ERR_ALIGN;
    const size_t need = qg::w8a8_dyn_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace) return QG_ERR_NULL;
        if (workspace_bytes < need) return QG_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return QG_ERR_ALIGN;
    }
    return QG_OK;
}

qg_status qgemm_w8a8_fp8_dynamic(const uint16_t* a_bf16, const uint8_t* w_e4m3, const float* w_scale,
                                 uint16_t* y_bf16, int M, int N, int K, void* workspace,
                                 size_t workspace_bytes, qg_stream stream) {
    if (!shape_ok(M, N, K)) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    const qg_status st = dynamic_args_ok(a_bf16, w_e4m3, w_scale, y_bf16, M, N, K, workspace, workspace_bytes);
    if (st != QG_OK) return st;
    qg::launch_qgemm_w8a8_fp8_dyn(a_bf16, w_e4m3, w_scale, y_bf16, M, N, K, workspace, as_stream(stream));
    return launched();
}

qg_status qgemm_w8a8_int8_dynamic(const uint16_t* a_bf16, const int8_t* w_i8, const float* w_scale,
                                  uint16_t* y_bf16, int M, int N, int K, void* workspace,
                                  size_t workspace_bytes, qg_stream stream) {
    if (!shape_ok(M, N, K) || K > kMaxKInt8) return QG_ERR_SHAPE;
    if (M == 0) return QG_OK;
    const qg_status st = dynamic_args_ok(a_bf16, w_i8, w_scale, y_bf16, M, N, K, workspace, workspace_bytes);
    if (st != QG_OK) return st;
    qg::launch_qgemm_w8a8_i8_dyn(a_bf16, w_i8, w_scale, y_bf16, M, N, K, workspace, as_stream(stream));
    return launched();
}

}  // extern "C"
