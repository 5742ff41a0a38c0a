// quant.hip - act_quant on gfx950.
//
// Per 128-element block of the last dimension: amax = max |x|, scale =
// max(amax, floor) / 448, codes = e4m3(x / scale) with the fp32 quotient
// correctly rounded ("Data flow - deepseek-ai/DeepSeek-V3", FP8 quantization
// bullet; pyshine tour, "FP8 with per-block scales").
//
// Mapping: the [M, K] input is a flat run of M*K/128 independent blocks (the
// scale of block i is scales[i], because scales are [M, K/128] row-major).
// Eight lanes own one block: each lane loads 32 contiguous bytes (16 bf16),
// so a wave64 reads 2 KB of contiguous memory per step, and the block max is
// an xor butterfly over the 8 lanes.  Each lane writes its 16 codes as one
// 16-byte store; the group's first lane writes the scale.  The kernel is HBM
// bound (3.03 bytes per element); two independent blocks per lane are in
// flight per iteration to keep enough loads outstanding.
//
// Quotient: fl(x / s) is needed only up to which e4m3 rounding interval it
// falls in.  y = x * fl(1/s) is within 3 ulp of fl(x/s); when y is more than
// 8 ulp away from every e4m3 rounding midpoint both land on the same code, so
// the exact IEEE division is only evaluated for lanes near a midpoint (and for
// quotients in the e4m3 subnormal range, below 2^-6).  The result equals
// encoding the correctly rounded quotient for every input.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

// fl(x / s) as far as e4m3 rounding can tell; r = fl(1 / s).
__device__ __forceinline__ float quotient_for_e4m3(float x, float s, float r) {
    float y = x * r;
    const uint32_t ay = __float_as_uint(y) & 0x7FFFFFFFu;
    const int d = (int)(ay & 0xFFFFFu) - 0x80000;
    const bool near_midpoint = (d >= -8) & (d <= 8);
    const bool small = (ay < 0x3C800000u) & (ay != 0u);
    if (near_midpoint | small) y = x / s;        // correctly rounded fp32 division
    return y;
}

template <bool kHw>
__device__ __forceinline__ void quant_block_part(const uint4 v0, const uint4 v1, int lane8,
                                                 uint4& out, float& scale) {
    float f[16];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    const float s = fmaxf(amax, kAmaxFloor) / kE4m3Max;  // correctly rounded
    const float r = 1.0f / s;
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quotient_for_e4m3(f[i], s, r);
    out.x = e4m3_encode4<kHw>(y[0], y[1], y[2], y[3]);
    out.y = e4m3_encode4<kHw>(y[4], y[5], y[6], y[7]);
    out.z = e4m3_encode4<kHw>(y[8], y[9], y[10], y[11]);
    out.w = e4m3_encode4<kHw>(y[12], y[13], y[14], y[15]);
    scale = s;
    (void)lane8;
}

// x: nblocks * 16 uint4 (256 B per block); q: nblocks * 8 uint4; s: nblocks floats.
template <bool kHw>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint4* __restrict__ x,
                                                        uint4* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t nblocks) {
    const int lane8 = threadIdx.x & 7;
    const int64_t groups = ((int64_t)gridDim.x * blockDim.x) >> 3;
    int64_t blk = (((int64_t)blockIdx.x * blockDim.x) + threadIdx.x) >> 3;
    // two blocks per iteration: blk and blk + groups
    for (; blk + groups < nblocks; blk += 2 * groups) {
        const uint4* p0 = x + blk * 16 + lane8 * 2;
        const uint4* p1 = x + (blk + groups) * 16 + lane8 * 2;
        const uint4 a0 = load_nt(p0);
        const uint4 a1 = load_nt(p0 + 1);
        const uint4 b0 = load_nt(p1);
        const uint4 b1 = load_nt(p1 + 1);
        uint4 qa, qb;
        float sa, sb;
        quant_block_part<kHw>(a0, a1, lane8, qa, sa);
        quant_block_part<kHw>(b0, b1, lane8, qb, sb);
        q[blk * 8 + lane8] = qa;
        q[(blk + groups) * 8 + lane8] = qb;
        if (lane8 == 0) {
            s[blk] = sa;
            s[blk + groups] = sb;
        }
    }
    if (blk < nblocks) {
        const uint4* p0 = x + blk * 16 + lane8 * 2;
        const uint4 a0 = load_nt(p0);
        const uint4 a1 = load_nt(p0 + 1);
        uint4 qa;
        float sa;
        quant_block_part<kHw>(a0, a1, lane8, qa, sa);
        q[blk * 8 + lane8] = qa;
        if (lane8 == 0) s[blk] = sa;
    }
}

// Encodes the fp32 bit patterns first .. first+count-1 (test helper).
template <bool kHw>
__global__ __launch_bounds__(256) void encode_range_kernel(uint32_t first, int64_t count,
                                                           uint8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float v = __uint_as_float(first + (uint32_t)i);
        uint32_t c;
        if constexpr (kHw) c = e4m3_encode2_hw(v, 0.0f) & 0xFFu;
        else c = e4m3_encode_sw(v);
        out[i] = (uint8_t)c;
    }
}

// The encoder act_quant uses.
constexpr bool kActQuantHwEncode = false;

hipError_t launch_act_quant(const void* x, void* q, float* s, int64_t M, int64_t K,
                            hipStream_t stream) {
    const int64_t nblocks = M * (K / kBlock);
    const int64_t wg_needed = (nblocks + 63) / 64;             // 32 blocks per WG-iteration, x2 unroll
    const int64_t wg_cap = (int64_t)device_cu_count() * 8;
    const int grid = (int)(wg_needed < wg_cap ? (wg_needed > 0 ? wg_needed : 1) : wg_cap);
    hipLaunchKernelGGL(act_quant_kernel<kActQuantHwEncode>, dim3(grid), dim3(256), 0, stream,
                       (const uint4*)x, (uint4*)q, s, nblocks);
    return hipGetLastError();
}

hipError_t launch_encode_range(uint32_t first, int64_t count, void* out, int variant,
                               hipStream_t stream) {
    const int64_t wg_needed = (count + 255) / 256;
    const int64_t wg_cap = (int64_t)device_cu_count() * 16;
    const int grid = (int)(wg_needed < wg_cap ? (wg_needed > 0 ? wg_needed : 1) : wg_cap);
    if (variant == 0) {
        if (kActQuantHwEncode)
            hipLaunchKernelGGL(encode_range_kernel<true>, dim3(grid), dim3(256), 0, stream, first,
                               count, (uint8_t*)out);
        else
            hipLaunchKernelGGL(encode_range_kernel<false>, dim3(grid), dim3(256), 0, stream, first,
                               count, (uint8_t*)out);
    } else {
        if (kActQuantHwEncode)
            hipLaunchKernelGGL(encode_range_kernel<false>, dim3(grid), dim3(256), 0, stream, first,
                               count, (uint8_t*)out);
        else
            hipLaunchKernelGGL(encode_range_kernel<true>, dim3(grid), dim3(256), 0, stream, first,
                               count, (uint8_t*)out);
    }
    return hipGetLastError();
}

}  // namespace bfp8
