// dequant.hip - weight_dequant on gfx950.
//
// out[n, k] = bf16( fp32( e4m3(w[n, k]) * s[n/128, k/128] ) ): the pages'
// route from an FP8 weight to an ordinary BF16 matmul (pyshine tour, "FP8
// with per-block scales"), also what the offline fp8->bf16 conversion does to
// each 1-byte tensor with its scale ("Behavior traces", fp8->bf16 trace).
//
// Vector kernel (K % 8 == 0, N*K a multiple of 1024, 8-byte aligned codes,
// 16-byte aligned output): fully contiguous 512-byte loads and 1 KB stores per
// wave instruction (see dequant_vec_kernel), so the kernel streams 3 bytes
// per element.  The gfx950 packed fp8 -> fp32 conversion decodes, one fp32
// multiply applies the block scale, and the packed fp32 -> bf16 conversion
// rounds to nearest even.  Scalar kernel: one element per lane for any other
// shape or alignment.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

// Eight codes (two dwords) -> eight bf16 (one 16-byte store), one scale.
__device__ __forceinline__ uint4 dequant8(uint32_t w0, uint32_t w1, float s) {
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

__device__ __forceinline__ uint2 load_nt8(const uint2* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    return make_uint2(v.x, v.y);
}

// A wave's unit of work is 1 KB of codes -> 2 KB of bf16.  Lane l converts
// the 8 codes at 8 l and the 8 codes at 512 + 8 l and stores 16 bytes at 16 l
// and at 1024 + 16 l, so every load instruction reads 512 contiguous bytes and
// every store instruction writes 1 KB contiguous bytes.  Eight codes never
// straddle a 128-wide scale block (8 divides 128).
// units = N * K / 1024 (< 2^31); kc = K / 8 (8-code groups per row); kb = ceil(K / 128).
__global__ __launch_bounds__(256) void dequant_vec_kernel(const uint2* __restrict__ w,
                                                          const float* __restrict__ s,
                                                          uint4* __restrict__ out,
                                                          uint32_t units, uint32_t kc,
                                                          uint32_t kb) {
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t waves = (gridDim.x * blockDim.x) >> 6;
    for (uint32_t u = wave; u < units; u += waves) {
        const uint32_t g0 = u * 128 + lane;          // 8-code group index
        const uint32_t g1 = g0 + 64;
        const uint2 v0 = load_nt8(w + g0);
        const uint2 v1 = load_nt8(w + g1);
        const uint32_t n0 = g0 / kc, n1 = g1 / kc;
        const uint32_t k0 = g0 - n0 * kc, k1 = g1 - n1 * kc;
        const float s0 = s[(n0 >> 7) * kb + (k0 >> 4)];
        const float s1 = s[(n1 >> 7) * kb + (k1 >> 4)];
        store_nt(out + g0, dequant8(v0.x, v0.y, s0));
        store_nt(out + g1, dequant8(v1.x, v1.y, s1));
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
    const bool vec = (K % 8 == 0) && (total % 1024 == 0) && (((uintptr_t)w & 7u) == 0) &&
                     (((uintptr_t)out & 15u) == 0) && (total / 1024 < ((int64_t)1 << 31)) &&
                     (total / 8 < ((int64_t)1 << 32));
    // a grid that covers the whole tensor at once: against a grid capped at 8
    // workgroups per CU (each wave looping over 16 units), [18432, 7168] took
    // 62.9 instead of 69.7 us from HBM; two units per wave were slower
    const int64_t cap = (int64_t)1 << 30;
    if (vec) {
        const int64_t units = total / 1024;                 // one unit per wave step
        const int64_t need = (units + 3) / 4;                // 4 waves per workgroup
        const int grid = (int)(need < cap ? (need > 0 ? need : 1) : cap);
        hipLaunchKernelGGL(dequant_vec_kernel, dim3(grid), dim3(256), 0, stream, (const uint2*)w,
                           s, (uint4*)out, (uint32_t)units, (uint32_t)(K / 8),
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
