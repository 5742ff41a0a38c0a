// internal.hpp - launchers behind the C ABI (include/bfp8.h).  Each launcher
// assumes its arguments were validated by the ABI layer and only enqueues
// kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bfp8 {

// Largest number of local experts the MoE dispatch handles (LDS counters).
constexpr int kMoeMaxGroups = 1024;

// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_act_quant(const void* x, void* q, float* s, int64_t M, int64_t K,
                            hipStream_t stream);
hipError_t launch_act_quant_pow2(const void* x, void* q, float* s, int64_t M, int64_t K,
                                 hipStream_t stream);
hipError_t launch_gemm_ue8m0(const void* a, const float* as, const void* b, const float* bs,
                             void* c, int64_t M, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
size_t gemm_ue8m0_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_act_quant_rows(const void* x, int64_t T, const int32_t* row_token,
                                 const int32_t* num_rows, void* q, float* s, int64_t M, int64_t K,
                                 hipStream_t stream);
hipError_t launch_encode_range(uint32_t first, int64_t count, void* out, int variant,
                               hipStream_t stream);
hipError_t launch_bf16_round_range(uint32_t first, int64_t count, void* out, int variant,
                                   hipStream_t stream);
hipError_t launch_weight_dequant(const void* w, const float* s, void* out, int64_t N, int64_t K,
                                 hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// The split last round of large GEMMs on 256 x 256 tiles (the fp8, power-of-two
// scale and bf16 GEMMs share it): when the tiles fill whole rounds of the 256 CUs
// and a last round at most half full of whole tile columns, the nt_tail last
// columns of tiles run as `splits` K ranges of kb_per 128-wide blocks each into
// an fp32 workspace [splits][M][N - 256 nt_main], then one ordered reduction.
struct TailPlan {
    int nt_main = 0, nt_tail = 0, splits = 0;
    int64_t kb_per = 0;
};
TailPlan tail_plan(int64_t M, int64_t N, int64_t K);
size_t tail_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Adds the K ranges' partial sums in order and writes bf16 columns [n1, N) of c.
hipError_t launch_tail_reduce(const float* ws, void* c, int64_t M, int64_t N, int64_t n1,
                              int splits, hipStream_t stream);

enum class GemmConfig { kBig256x256, kBig256x128, kBig128x128 };
GemmConfig gemm_config(int64_t M, int64_t N, int64_t K);
const char* gemm_config_name(GemmConfig cfg);
hipError_t launch_gemm(const void* a, const float* as, const void* b, const float* bs, void* c,
                       int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
hipError_t launch_gemm_quant(const void* a, const float* as, const void* b, const float* bs,
                             void* q, float* qs, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream);
hipError_t launch_gemm_swiglu_quant(const void* a, const float* as, const void* w13,
                                    const float* s13, void* q, float* qs, int64_t M, int64_t n_out,
                                    int64_t K, hipStream_t stream);
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
// Size of the library-owned device scratch array behind the no-allocation GEMM
// entry point (one per GPU, resident until the process ends).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t launch_gemm_noalloc(const void* a, const float* as, const void* b, const float* bs,
                               void* c, int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_linear_fp8(const void* x, const void* b, const float* bs, void* c, int64_t M,
                             int64_t N, int64_t K, void* workspace, hipStream_t stream);
hipError_t launch_gemm_grouped(const void* a, const float* as, const void* b, const float* bs,
                               void* c, const int32_t* off, int32_t G, int64_t total_M,
                               int64_t N, int64_t K, hipStream_t stream);

hipError_t launch_gemm_bf16(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
const char* gemm_bf16_config_name(int64_t M, int64_t N, int64_t K);

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t G);
hipError_t launch_moe_dispatch(const int32_t* topk, int64_t T, int32_t k, int32_t lo, int32_t G,
                               int32_t* off, int32_t* row_token, int32_t* slot_row, void* ws,
                               hipStream_t stream);
hipError_t launch_moe_combine(const void* out, int64_t rows_cap, const int32_t* slot_row,
                              const float* weight, void* y, int64_t T, int32_t k, int64_t N,
                              hipStream_t stream);

}  // namespace bfp8
