// api.hip - the C ABI declared in include/bfp8.h: host-side validation, then
// one launcher call.  Validation touches no HIP API, so every error code can
// be exercised on a machine without a GPU.
#include <mutex>

#include "../../include/bfp8.h"
#include "internal.hpp"

namespace bfp8 {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

}  // namespace bfp8

namespace {

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? BFP8_OK : BFP8_ERR_HIP; }

}  // namespace

extern "C" {

int bfp8_version(void) { return BFP8_VERSION; }

// The fp8 GEMM tiles address a tile's rows with 32-bit byte offsets (row * K,
// row < 256), so K stays below 2^22 (the bf16 GEMM's limit too).
static bool gemm_k_ok(int64_t K) { return K > 0 && K % BFP8_BLOCK == 0 && K < ((int64_t)1 << 22); }

const char* bfp8_status_string(int status) {
    switch (status) {
        case BFP8_OK: return "ok";
        case BFP8_ERR_NULL: return "a required pointer is NULL";
        case BFP8_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 128, or a size past its stated limit)";
        case BFP8_ERR_ALIGN: return "pointer misaligned";
        case BFP8_ERR_WORKSPACE: return "workspace smaller than the matching *_workspace_size() call";
        case BFP8_ERR_GROUPS: return "group count out of range (below 1, or above the dispatch limit)";
        case BFP8_ERR_HIP: return "HIP runtime error at launch";
        case BFP8_ERR_ARG: return "invalid argument";
        case BFP8_ERR_SCRATCH: return "problem needs more scratch than the no-allocation entry point's fixed buffer holds";
        default: return "unknown status";
    }
}

int bfp8_act_quant(const void* x_bf16, void* q_e4m3, float* scales, int64_t M, int64_t K,
                   void* stream) {
    if (M < 0 || K <= 0 || K % BFP8_BLOCK != 0) return BFP8_ERR_SHAPE;
    if (M == 0) return BFP8_OK;
    if (!x_bf16 || !q_e4m3 || !scales) return BFP8_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4)) return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_act_quant(x_bf16, q_e4m3, scales, M, K, (hipStream_t)stream));
}

int bfp8_act_quant_ue8m0(const void* x_bf16, void* q_e4m3, float* scales, int64_t M, int64_t K,
                         void* stream) {
    if (M < 0 || K <= 0 || K % BFP8_BLOCK != 0) return BFP8_ERR_SHAPE;
    if (M == 0) return BFP8_OK;
    if (!x_bf16 || !q_e4m3 || !scales) return BFP8_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4)) return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_act_quant_pow2(x_bf16, q_e4m3, scales, M, K, (hipStream_t)stream));
}

size_t bfp8_gemm_ue8m0_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % BFP8_BLOCK != 0) return 0;
    return bfp8::gemm_ue8m0_workspace_bytes(M, N, K);
}

int bfp8_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s, void* c_bf16,
                    int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (M < 0 || N < 0 || !gemm_k_ok(K)) return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !b || !b_s || !c_bf16) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
        !aligned(c_bf16, 2))
        return BFP8_ERR_ALIGN;
    if (workspace) {
        if (!aligned(workspace, 16)) return BFP8_ERR_ALIGN;
        if (workspace_bytes < bfp8::gemm_ue8m0_workspace_bytes(M, N, K)) return BFP8_ERR_WORKSPACE;
    }
    return from_hip(bfp8::launch_gemm_ue8m0(a, a_s, b, b_s, c_bf16, M, N, K, workspace,
                                            workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

int bfp8_weight_dequant(const void* w_e4m3, const float* s, void* out_bf16, int64_t N, int64_t K,
                        void* stream) {
    if (N < 0 || K < 0) return BFP8_ERR_SHAPE;
    if (N == 0 || K == 0) return BFP8_OK;
    if (!w_e4m3 || !s || !out_bf16) return BFP8_ERR_NULL;
    if (!aligned(out_bf16, 2) || !aligned(s, 4)) return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_weight_dequant(w_e4m3, s, out_bf16, N, K, (hipStream_t)stream));
}

size_t bfp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % BFP8_BLOCK != 0) return 0;
    return bfp8::gemm_workspace_bytes(M, N, K);
}

int bfp8_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c_bf16,
              int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
              void* stream) {
    if (M < 0 || N < 0 || !gemm_k_ok(K)) return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !b || !b_s || !c_bf16) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
        !aligned(c_bf16, 2))
        return BFP8_ERR_ALIGN;
    if (workspace) {
        if (!aligned(workspace, 16)) return BFP8_ERR_ALIGN;
        if (workspace_bytes < bfp8::gemm_workspace_bytes(M, N, K)) return BFP8_ERR_WORKSPACE;
    }
    return from_hip(bfp8::launch_gemm(a, a_s, b, b_s, c_bf16, M, N, K, workspace,
                                      workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

int bfp8_gemm_noalloc(const void* a, const float* a_s, const void* b, const float* b_s,
                      void* c_bf16, int64_t M, int64_t N, int64_t K, void* stream) {
    static_assert(BFP8_NOALLOC_SCRATCH_BYTES == bfp8::kNoAllocScratchBytes, "scratch size");
    if (M < 0 || N < 0 || !gemm_k_ok(K)) return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !b || !b_s || !c_bf16) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
        !aligned(c_bf16, 2))
        return BFP8_ERR_ALIGN;
    if (bfp8::gemm_workspace_bytes(M, N, K) > BFP8_NOALLOC_SCRATCH_BYTES) return BFP8_ERR_SCRATCH;
    return from_hip(bfp8::launch_gemm_noalloc(a, a_s, b, b_s, c_bf16, M, N, K, (hipStream_t)stream));
}

int bfp8_gemm_act_quant(const void* a, const float* a_s, const void* b, const float* b_s,
                        void* q_e4m3, float* q_scales, int64_t M, int64_t N, int64_t K,
                        void* stream) {
    if (M < 0 || N < 0 || !gemm_k_ok(K) || N % BFP8_BLOCK != 0)
        return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !b || !b_s || !q_e4m3 || !q_scales) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
        !aligned(q_e4m3, 4) || !aligned(q_scales, 4))
        return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_gemm_quant(a, a_s, b, b_s, q_e4m3, q_scales, M, N, K,
                                            (hipStream_t)stream));
}

int bfp8_gemm_swiglu_act_quant(const void* a, const float* a_s, const void* w13,
                               const float* s13, void* q_e4m3, float* q_scales, int64_t M,
                               int64_t N, int64_t K, void* stream) {
    if (M < 0 || N < 0 || !gemm_k_ok(K) || N % BFP8_BLOCK != 0)
        return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !w13 || !s13 || !q_e4m3 || !q_scales) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(w13, 16) || !aligned(a_s, 4) || !aligned(s13, 4) ||
        !aligned(q_e4m3, 4) || !aligned(q_scales, 4))
        return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_gemm_swiglu_quant(a, a_s, w13, s13, q_e4m3, q_scales, M, N, K,
                                                   (hipStream_t)stream));
}

size_t bfp8_linear_fp8_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % BFP8_BLOCK != 0) return 0;
    return bfp8::linear_workspace_bytes(M, N, K);
}

int bfp8_linear_fp8(const void* x_bf16, const void* w, const float* w_s, void* y_bf16, int64_t M,
                    int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || !gemm_k_ok(K)) return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!x_bf16 || !w || !w_s || !y_bf16 || !workspace) return BFP8_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(w, 16) || !aligned(w_s, 4) || !aligned(y_bf16, 2) ||
        !aligned(workspace, 256))
        return BFP8_ERR_ALIGN;
    if (workspace_bytes < bfp8::linear_workspace_bytes(M, N, K)) return BFP8_ERR_WORKSPACE;
    return from_hip(bfp8::launch_linear_fp8(x_bf16, w, w_s, y_bf16, M, N, K, workspace,
                                            (hipStream_t)stream));
}

int bfp8_gemm_grouped(const void* a, const float* a_s, const void* b, const float* b_s,
                      void* c_bf16, const int32_t* group_offsets, int32_t G, int64_t total_M,
                      int64_t N, int64_t K, void* stream) {
    if (total_M < 0 || N < 0 || !gemm_k_ok(K)) return BFP8_ERR_SHAPE;
    if (G < 1) return BFP8_ERR_GROUPS;
    if (total_M == 0 || N == 0) return BFP8_OK;
    if (!a || !a_s || !b || !b_s || !c_bf16 || !group_offsets) return BFP8_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(a_s, 4) || !aligned(b_s, 4) ||
        !aligned(c_bf16, 2) || !aligned(group_offsets, 4))
        return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_gemm_grouped(a, a_s, b, b_s, c_bf16, group_offsets, G, total_M,
                                              N, K, (hipStream_t)stream));
}

size_t bfp8_gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % 64 != 0) return 0;
    return bfp8::tail_workspace_bytes(M, N, K);
}

int bfp8_gemm_bf16(const void* a_bf16, const void* b_bf16, void* c_bf16, int64_t M, int64_t N,
                   int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || K >= ((int64_t)1 << 22)) return BFP8_ERR_SHAPE;
    if (M == 0 || N == 0) return BFP8_OK;
    if (!a_bf16 || !b_bf16 || !c_bf16) return BFP8_ERR_NULL;
    if (!aligned(a_bf16, 16) || !aligned(b_bf16, 16) || !aligned(c_bf16, 2)) return BFP8_ERR_ALIGN;
    if (workspace) {
        if (!aligned(workspace, 16)) return BFP8_ERR_ALIGN;
        if (workspace_bytes < bfp8::tail_workspace_bytes(M, N, K)) return BFP8_ERR_WORKSPACE;
    }
    return from_hip(bfp8::launch_gemm_bf16(a_bf16, b_bf16, c_bf16, M, N, K, workspace,
                                           workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

size_t bfp8_moe_dispatch_workspace_size(int64_t T, int32_t k, int32_t G) {
    if (T <= 0 || k < 1 || G < 1 || G > BFP8_MOE_MAX_GROUPS || T * (int64_t)k >= ((int64_t)1 << 31))
        return 0;
    return bfp8::moe_dispatch_workspace_bytes(T, k, G);
}

int bfp8_moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t expert_lo,
                      int32_t G, int32_t* group_offsets, int32_t* row_token, int32_t* slot_row,
                      void* workspace, size_t workspace_bytes, void* stream) {
    static_assert(BFP8_MOE_MAX_GROUPS == bfp8::kMoeMaxGroups, "dispatch group limit");
    if (T < 0 || k < 1 || T * (int64_t)k >= ((int64_t)1 << 31)) return BFP8_ERR_SHAPE;
    if (G < 1 || G > BFP8_MOE_MAX_GROUPS) return BFP8_ERR_GROUPS;
    const size_t need = T > 0 ? bfp8::moe_dispatch_workspace_bytes(T, k, G) : 0;
    if (!group_offsets) return BFP8_ERR_NULL;
    if (T > 0 && (!topk_idx || !row_token || !slot_row || !workspace)) return BFP8_ERR_NULL;
    if (!aligned(group_offsets, 4) || !aligned(topk_idx, 4) || !aligned(row_token, 4) ||
        !aligned(slot_row, 4) || !aligned(workspace, 4))
        return BFP8_ERR_ALIGN;
    if (workspace_bytes < need) return BFP8_ERR_WORKSPACE;
    return from_hip(bfp8::launch_moe_dispatch(topk_idx, T, k, expert_lo, G, group_offsets,
                                              row_token, slot_row, workspace,
                                              (hipStream_t)stream));
}

int bfp8_act_quant_rows(const void* x_bf16, int64_t T, const int32_t* row_token,
                        const int32_t* num_rows, void* q_e4m3, float* scales, int64_t M,
                        int64_t K, void* stream) {
    if (T < 0 || M < 0 || K <= 0 || K % BFP8_BLOCK != 0) return BFP8_ERR_SHAPE;
    if (M == 0) return BFP8_OK;
    if ((T > 0 && !x_bf16) || !row_token || !q_e4m3 || !scales) return BFP8_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(scales, 4) ||
        !aligned(row_token, 4) || !aligned(num_rows, 4))
        return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_act_quant_rows(x_bf16, T, row_token, num_rows, q_e4m3, scales, M,
                                                K, (hipStream_t)stream));
}

int bfp8_moe_combine(const void* expert_out_bf16, int64_t rows, const int32_t* slot_row,
                     const float* weights, void* y_bf16, int64_t T, int32_t k, int64_t N,
                     void* stream) {
    if (T < 0 || k < 1 || N < 0 || rows < 0 || T > ((int64_t)1 << 24) ||
        T * (int64_t)k >= ((int64_t)1 << 31) || (N + 2047) / 2048 > 65535)
        return BFP8_ERR_SHAPE;
    if (T == 0 || N == 0) return BFP8_OK;
    if ((rows > 0 && !expert_out_bf16) || !slot_row || !weights || !y_bf16) return BFP8_ERR_NULL;
    if (!aligned(expert_out_bf16, 2) || !aligned(y_bf16, 2) || !aligned(slot_row, 4) ||
        !aligned(weights, 4))
        return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_moe_combine(expert_out_bf16, rows, slot_row, weights, y_bf16, T,
                                             k, N, (hipStream_t)stream));
}

const char* bfp8_gemm_kernel_name(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0 || K % BFP8_BLOCK != 0) return "none";
    return bfp8::gemm_config_name(bfp8::gemm_config(M, N, K));
}

int bfp8_e4m3_encode_range(uint32_t first, int64_t count, void* out, int variant, void* stream) {
    if (count < 0 || (uint64_t)first + (uint64_t)count > (uint64_t)1 << 32) return BFP8_ERR_SHAPE;
    if (variant != 0 && variant != 1) return BFP8_ERR_ARG;
    if (count == 0) return BFP8_OK;
    if (!out) return BFP8_ERR_NULL;
    return from_hip(bfp8::launch_encode_range(first, count, out, variant, (hipStream_t)stream));
}

int bfp8_bf16_round_range(uint32_t first, int64_t count, void* out, int variant, void* stream) {
    if (count < 0 || (uint64_t)first + (uint64_t)count > (uint64_t)1 << 32) return BFP8_ERR_SHAPE;
    if (variant != 0 && variant != 1) return BFP8_ERR_ARG;
    if (count == 0) return BFP8_OK;
    if (!out) return BFP8_ERR_NULL;
    if (!aligned(out, 2)) return BFP8_ERR_ALIGN;
    return from_hip(bfp8::launch_bf16_round_range(first, count, out, variant, (hipStream_t)stream));
}

}  // extern "C"
