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
// bound (3.03 bytes per element).  The grid covers every block at once (one
// block per eight lanes; the loop only matters past 2^35 blocks): against a
// grid capped at 16 workgroups per CU with two blocks per lane per iteration,
// [8192, 7168] took 29.6 instead of 32.9 us (inputs in the Infinity Cache)
// and 31.8 instead of 35.0 us (from HBM), [8192, 18432] 78.9 instead of 91.5
// us from HBM; four blocks per lane per iteration were slower still.
//
// Per element the work is: widen bf16, one max, a three-operation correctly
// rounded quotient (see quotient()), and the gfx950 fp32 -> e4m3 conversion
// after a clamp to +-448 (proven equal to the oracle's encoder on all 2^32
// fp32 inputs by the GPU tests).  The two divisions per block (scale and its
// reciprocal) are shared by the 8 lanes of the block.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

// Power-of-two scale (the e8m0 reading of the model's scale_fmt): the scale
// max(amax, floor) / 448 rounded up to the next power of two, taken from its
// fp32 bits (biased exponent, plus one when any mantissa bit is set).  The
// quotient by it is then an exact scaling.
__device__ __forceinline__ float pow2_ceil(float y) {
    uint32_t e = __float_as_uint(y) >> 23;
    if (__float_as_uint(y) & 0x7FFFFFu) e += 1;
    return __uint_as_float(e << 23);
}

template <bool kHw, bool kPow2 = false>
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
    for (int i = 0; i < 16; i += 2) amax = fmaxf(amax, fmaxf(fabsf(f[i]), fabsf(f[i + 1])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    float s = fmaxf(amax, kAmaxFloor) / kE4m3Max;        // correctly rounded
    if (kPow2) s = pow2_ceil(s);
    const float r = 1.0f / s;
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quotient(f[i], s, r);
    out.x = e4m3_encode4<kHw>(y[0], y[1], y[2], y[3]);
    out.y = e4m3_encode4<kHw>(y[4], y[5], y[6], y[7]);
    out.z = e4m3_encode4<kHw>(y[8], y[9], y[10], y[11]);
    out.w = e4m3_encode4<kHw>(y[12], y[13], y[14], y[15]);
    scale = s;
    (void)lane8;
}

// x: nblocks * 16 uint4 (256 B per block); q: nblocks * 8 uint4; s: nblocks floats.
template <bool kHw, bool kPow2 = false>
__global__ __launch_bounds__(256) void act_quant_kernel(const uint4* __restrict__ x,
                                                        uint4* __restrict__ q,
                                                        float* __restrict__ s,
                                                        int64_t nblocks) {
    const int lane8 = threadIdx.x & 7;
    const int64_t groups = ((int64_t)gridDim.x * blockDim.x) >> 3;
    for (int64_t blk = (((int64_t)blockIdx.x * blockDim.x) + threadIdx.x) >> 3; blk < nblocks;
         blk += groups) {
        const uint4* p0 = x + blk * 16 + lane8 * 2;
        const uint4 a0 = load_nt(p0);
        const uint4 a1 = load_nt(p0 + 1);
        uint4 qa;
        float sa;
        quant_block_part<kHw, kPow2>(a0, a1, lane8, qa, sa);
        q[blk * 8 + lane8] = qa;
        if (lane8 == 0) s[blk] = sa;
    }
}

// act_quant of gathered rows: output row r is the quantization of input row
// row_token[r], for r < min(*num_rows, M); rows past that, and rows whose
// token lies outside [0, T), are not written.  Quantization is row-local, so
// this equals gathering rows of act_quant(x).  Same mapping as
// act_quant_kernel (eight lanes per 128-element block, a grid covering every
// block); the block index splits into (output row, k-block) and the source
// block is (row_token[row], k-block).
__device__ __forceinline__ bool rows_source(const uint4* __restrict__ x,
                                            const int32_t* __restrict__ row_token, int64_t T,
                                            int64_t KB, int64_t blk, const uint4*& src) {
    const int64_t r = blk / KB;
    const int64_t kb = blk - r * KB;
    const int64_t tok = row_token[r];
    if (tok < 0 || tok >= T) return false;
    src = x + (tok * KB + kb) * 16;
    return true;
}

template <bool kHw>
__global__ __launch_bounds__(256) void act_quant_rows_kernel(
    const uint4* __restrict__ x, int64_t T, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ num_rows, uint4* __restrict__ q, float* __restrict__ s, int64_t M,
    int64_t KB) {
    int64_t rows = M;
    if (num_rows) {
        const int64_t nr = *num_rows;
        rows = nr < 0 ? 0 : (nr < M ? nr : M);
    }
    const int64_t nblocks = rows * KB;
    const int lane8 = threadIdx.x & 7;
    const int64_t groups = ((int64_t)gridDim.x * blockDim.x) >> 3;
    for (int64_t blk = (((int64_t)blockIdx.x * blockDim.x) + threadIdx.x) >> 3; blk < nblocks;
         blk += groups) {
        const uint4* pa = nullptr;
        if (rows_source(x, row_token, T, KB, blk, pa)) {
            const uint4 a0 = load_nt(pa + lane8 * 2);
            const uint4 a1 = load_nt(pa + lane8 * 2 + 1);
            uint4 qa;
            float sa;
            quant_block_part<kHw>(a0, a1, lane8, qa, sa);
            q[blk * 8 + lane8] = qa;
            if (lane8 == 0) s[blk] = sa;
        }
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

// Rounds the fp32 bit patterns first .. first+count-1 to bf16 with the
// packed conversion the dequant and GEMM epilogues use (variant 0) or with the
// bit rule (variant 1) (test helper).
template <bool kHw>
__global__ __launch_bounds__(256) void bf16_round_range_kernel(uint32_t first, int64_t count,
                                                               uint16_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const float v = __uint_as_float(first + (uint32_t)i);
        uint32_t h;
        if constexpr (kHw) h = pack_bf16x2(v, 0.0f) & 0xFFFFu;
        else h = bf16_rne_bits(v);
        out[i] = (uint16_t)h;
    }
}

hipError_t launch_bf16_round_range(uint32_t first, int64_t count, void* out, int variant,
                                   hipStream_t stream) {
    const int64_t wg_needed = (count + 255) / 256;
    const int64_t wg_cap = (int64_t)device_cu_count() * 16;
    const int grid = (int)(wg_needed < wg_cap ? (wg_needed > 0 ? wg_needed : 1) : wg_cap);
    if (variant == 0)
        hipLaunchKernelGGL(bf16_round_range_kernel<true>, dim3(grid), dim3(256), 0, stream, first,
                           count, (uint16_t*)out);
    else
        hipLaunchKernelGGL(bf16_round_range_kernel<false>, dim3(grid), dim3(256), 0, stream, first,
                           count, (uint16_t*)out);
    return hipGetLastError();
}

// The encoder act_quant uses.
constexpr bool kActQuantHwEncode = true;

// Workgroups (256 lanes, 32 blocks) that cover n blocks at once; past 2^30
// workgroups the kernels loop.
static int quant_grid(int64_t nblocks) {
    const int64_t need = (nblocks + 31) / 32;
    const int64_t cap = (int64_t)1 << 30;
    return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

hipError_t launch_act_quant(const void* x, void* q, float* s, int64_t M, int64_t K,
                            hipStream_t stream) {
    const int64_t nblocks = M * (K / kBlock);
    const int grid = quant_grid(nblocks);
    hipLaunchKernelGGL(act_quant_kernel<kActQuantHwEncode>, dim3(grid), dim3(256), 0, stream,
                       (const uint4*)x, (uint4*)q, s, nblocks);
    return hipGetLastError();
}

hipError_t launch_act_quant_rows(const void* x, int64_t T, const int32_t* row_token,
                                 const int32_t* num_rows, void* q, float* s, int64_t M, int64_t K,
                                 hipStream_t stream) {
    const int64_t KB = K / kBlock;
    const int64_t nblocks = M * KB;                            // upper bound: *num_rows may be less
    // M is a capacity that the rows on the device may fill only in part, so the grid
    // stops at 32 workgroups per CU and loops: with room for 65536 rows and 8195 used
    // ([8192, 7168] source) that took 33.0 us against 53.4 for a grid covering the
    // capacity and 36.2 for 16 per CU with two blocks per lane; 33.1 against 34.2 us
    // with exactly 8195 rows
    int grid = quant_grid(nblocks);
    const int cap = (int)device_cu_count() * 32;
    grid = grid < cap ? grid : cap;
    hipLaunchKernelGGL(act_quant_rows_kernel<kActQuantHwEncode>, dim3(grid), dim3(256), 0, stream,
                       (const uint4*)x, T, row_token, num_rows, (uint4*)q, s, M, KB);
    return hipGetLastError();
}

hipError_t launch_act_quant_pow2(const void* x, void* q, float* s, int64_t M, int64_t K,
                                 hipStream_t stream) {
    const int64_t nblocks = M * (K / kBlock);
    const int grid = quant_grid(nblocks);
    hipLaunchKernelGGL((act_quant_kernel<kActQuantHwEncode, true>), dim3(grid), dim3(256), 0, stream,
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
