// device_codec.hpp - e4m3 / bf16 conversions used inside the gfx950 kernels.
//
// e4m3 is the OCP FP8 E4M3 format (torch.float8_e4m3fn): s.eeee.mmm, bias 7,
// no infinities, NaN only at S.1111.111, largest finite magnitude 448 (0x7E),
// the "e4m3 ceiling" of the pyshine DeepSeek-V3 tour ("FP8 with per-block
// scales").  Quantization rounds to nearest, ties to even, and saturates at
// +-448; the sign of zero is kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

constexpr int kBlock = 128;
constexpr float kE4m3Max = 448.0f;
// Lower clamp on a block's max |x| before dividing by 448 (the reading of
// "clamping each tile's max": keeps the scale positive on all-zero blocks).
constexpr float kAmaxFloor = 1e-4f;

// Software encoder: integer rounding of the fp32 bit pattern.
//   |v| >= 448        -> 0x7E (saturate; also +-inf)
//   |v| <  2^-6       -> round(|v| * 2^9) with ties to even: subnormal codes 0..8
//   otherwise         -> keep 3 mantissa bits, round the dropped 20 bits to
//                        nearest-even, re-bias the exponent from 127 to 7
__device__ __forceinline__ uint32_t e4m3_encode_sw(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a > 0x7F800000u) {
        code = 0x7Fu;                                   // NaN in, NaN out
    } else if (a >= 0x43E00000u) {                      // 448.0f
        code = 0x7Eu;
    } else if (a < 0x3C800000u) {                       // 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    }
    return sign | code;
}

// Hardware encoder: clamp to +-448, then the gfx950 fp32 -> OCP-e4m3
// conversion (round to nearest even).  Packs two codes into the low 16 bits.
__device__ __forceinline__ uint32_t e4m3_encode2_hw(float v0, float v1) {
    v0 = __builtin_amdgcn_fmed3f(v0, -kE4m3Max, kE4m3Max);
    v1 = __builtin_amdgcn_fmed3f(v1, -kE4m3Max, kE4m3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false) & 0xFFFFu;
}

// Four codes into one dword (byte i = code of v[i]).
template <bool kHw>
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
    if constexpr (kHw) {
        v0 = __builtin_amdgcn_fmed3f(v0, -kE4m3Max, kE4m3Max);
        v1 = __builtin_amdgcn_fmed3f(v1, -kE4m3Max, kE4m3Max);
        v2 = __builtin_amdgcn_fmed3f(v2, -kE4m3Max, kE4m3Max);
        v3 = __builtin_amdgcn_fmed3f(v3, -kE4m3Max, kE4m3Max);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
        return (uint32_t)w;
    } else {
        return e4m3_encode_sw(v0) | (e4m3_encode_sw(v1) << 8) | (e4m3_encode_sw(v2) << 16) |
               (e4m3_encode_sw(v3) << 24);
    }
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16 (low half = a), round to nearest even.  gfx950 has a
// native packed conversion; written as the bit rule so the result does not
// depend on instruction selection:
//   keep the upper 16 bits, add one ulp when the dropped half exceeds one half
//   or equals it with an odd kept part.  NaN -> quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2_sw(float a, float b) {
    return bf16_rne_bits(a) | (bf16_rne_bits(b) << 16);
}

// The same rounding by the gfx950 packed conversion (v_cvt_pk_bf16_f32,
// round to nearest even); the GPU tests compare it with the bit rule above
// and with the oracle on every fp32 input.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Decode of a packed pair of e4m3 codes (bytes 0-1 or 2-3 of w) by the gfx950
// conversion; every e4m3 value is exact in fp32.
template <bool kHi>
__device__ __forceinline__ void e4m3_decode2(uint32_t w, float& f0, float& f1) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f r = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
    f0 = r.x;
    f1 = r.y;
}

// 16-byte loads and stores with the non-temporal hint (streamed data that is
// touched once).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4* p, const uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4*)p);
}

// Correctly rounded fp32 quotient x / s from the correctly rounded reciprocal
// r = fl(1 / s): y0 = fl(x r) is within one ulp of x / s, the remainder
// x - y0 s is exact as one fused multiply-add, and one more fused step
// y0 + (x - y0 s) r rounds to fl(x / s) (Markstein's correction step).  The
// GPU tests check the kernel against the oracle's fp32 division on every pair
// of bf16 block maximum and bf16 element.
// The correction step turns a quotient of -0 into +0 (-0 + +0 rounds to +0),
// so the sign of x is put back; for x != 0 it is already the quotient's sign
// because s > 0.
__device__ __forceinline__ float quotient(float x, float s, float r) {
    const float y0 = x * r;
    const float e = __builtin_fmaf(-y0, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, y0), x);
}

// An fp32 value rounded to bf16 (nearest even, the conversion every bf16
// output uses) and widened back.
__device__ __forceinline__ float bf16_round_f32(float x) {
    return __uint_as_float((pack_bf16x2(x, x) & 0xFFFFu) << 16);
}

}  // namespace bfp8
