// dequant.hip - weight_dequant on gfx950.
//
// out[n, k] = bf16( fp32( e4m3(w[n, k]) * s[n/128, k/128] ) ): the pages'
// route from an FP8 weight to an ordinary BF16 matmul (pyshine tour, "FP8
// with per-block scales"), also what the offline fp8->bf16 conversion does to
// each 1-byte tensor with its scale ("Behavior traces", fp8->bf16 trace).
//
// Vector kernel (K % 16 == 0, 16-byte aligned w and out): each lane turns one
// 16-byte chunk of codes (16 elements, inside one 128-wide scale block) into
// two 16-byte bf16 stores, so the kernel streams 3 bytes per element at HBM
// rate.  The gfx950 packed fp8 -> fp32 conversion decodes, one fp32 multiply
// applies the block scale, and the bf16 rounding is the nearest-even bit rule.
// Scalar kernel: one element per lane for any other shape or alignment.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

__device__ __forceinline__ uint4 dequant16_lo(uint32_t w0, uint32_t w1, float s) {
    float f[8];
    e4m3_decode2<false>(w0, f[0], f[1]);
    e4m3_decode2<true>(w0, f[2], f[3]);
    e4m3_decode2<false>(w1, f[4], f[5]);
    e4m3_decode2<true>(w1, f[6], f[7]);
    uint4 o;
    o.x = pack_bf16x2(f[0] * s, f[1] * s);
    o.y = pack_bf16x2(f[2] * s, f[3] * s);
    o.z = pack_bf16x2(f[4] * s, f[5] * s);
    o.w = pack_bf16x2(f[6] * s, f[7] * s);
    return o;
}

// chunks = N * K / 16 (< 2^31); kc = K / 16; kb = ceil(K / 128).
__global__ __launch_bounds__(256) void dequant_vec_kernel(const uint4* __restrict__ w,
                                                          const float* __restrict__ s,
                                                          uint4* __restrict__ out,
                                                          uint32_t chunks, uint32_t kc,
                                                          uint32_t kb) {
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
        const uint4 v = load_nt(w + c);
        const uint32_t n = c / kc;
        const uint32_t k16 = c - n * kc;
        const float sc = s[(n >> 7) * kb + (k16 >> 3)];
        const uint4 o0 = dequant16_lo(v.x, v.y, sc);
        const uint4 o1 = dequant16_lo(v.z, v.w, sc);
        store_nt(out + 2 * (size_t)c, o0);
        store_nt(out + 2 * (size_t)c + 1, o1);
    }
}

__global__ __launch_bounds__(256) void dequant_scalar_kernel(const uint8_t* __restrict__ w,
                                                             const float* __restrict__ s,
                                                             uint16_t* __restrict__ out,
                                                             int64_t N, int64_t K) {
    const int64_t total = N * K;
    const int64_t kb = (K + kBlock - 1) / kBlock;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t n = i / K, k = i - n * K;
        float f0, f1;
        e4m3_decode2<false>((uint32_t)w[i], f0, f1);
        out[i] = (uint16_t)bf16_rne_bits(f0 * s[(n / kBlock) * kb + k / kBlock]);
    }
}

hipError_t launch_weight_dequant(const void* w, const float* s, void* out, int64_t N, int64_t K,
                                 hipStream_t stream) {
    const int64_t total = N * K;
    const bool vec = (K % 16 == 0) && (((uintptr_t)w & 15u) == 0) &&
                     (((uintptr_t)out & 15u) == 0) && (total / 16 < ((int64_t)1 << 31));
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (vec) {
        const int64_t chunks = total / 16;
        const int64_t need = (chunks + 255) / 256;
        const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
        hipLaunchKernelGGL(dequant_vec_kernel, dim3(grid), dim3(256), 0, stream, (const uint4*)w,
                           s, (uint4*)out, (uint32_t)chunks, (uint32_t)(K / 16),
                           (uint32_t)((K + kBlock - 1) / kBlock));
    } else {
        const int64_t need = (total + 255) / 256;
        const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
        hipLaunchKernelGGL(dequant_scalar_kernel, dim3(grid), dim3(256), 0, stream,
                           (const uint8_t*)w, s, (uint16_t*)out, N, K);
    }
    return hipGetLastError();
}

}  // namespace bfp8
