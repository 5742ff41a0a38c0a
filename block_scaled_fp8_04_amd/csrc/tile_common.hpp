// tile_common.hpp - pieces shared by the large-tile GEMM kernels on gfx950:
// MFMA operand types, the LDS row swizzle, fragment assembly, counted waits,
// the LDS-only barrier and direct-to-LDS buffer loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// LDS chunk swizzle of a 128-byte row: logical 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r).  Measured on MI355X with the fragment
// read pattern (16 rows x one chunk per 16 lanes), xor-ing with (r & 7) alone,
// or with ((r >> 1) & 7), leaves two-way bank conflicts; additionally flipping
// the low bit for rows 8..15 of each 16-row group removes them.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ v8i frag_from(const uint4 x0, const uint4 x1) {
    v8i f;
    f[0] = (int)x0.x; f[1] = (int)x0.y; f[2] = (int)x0.z; f[3] = (int)x0.w;
    f[4] = (int)x1.x; f[5] = (int)x1.y; f[6] = (int)x1.z; f[7] = (int)x1.w;
    return f;
}

template <int S>
struct StageId {
    static constexpr int value = S;
};

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef const __attribute__((address_space(1))) void* gbl_void_t;

// s_waitcnt that waits only for vmcnt <= n (gfx9 encoding: vmcnt[3:0] in bits
// 3:0 and vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Workgroup barrier whose memory fence covers LDS only: outstanding global
// loads are not waited for here (the direct-to-LDS loads are counted with
// wait_vmcnt by each wave before it arrives).
// The empty asm statements are compiler-only memory barriers (they emit no
// instruction) so that no LDS access is moved across the hardware barrier.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Direct-to-LDS loads through a buffer resource (MUBUF).  Unlike the flat
// global form, the compiler tracks these only with the vector-memory
// counter, so LDS reads that follow them keep precise LDS waits.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const int num = (int)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num, 0x00020000);
}
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)lds_dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf_lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)lds_dst, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ void load_lds16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)lds_dst, 4, 0, 0);
}

// the same with the non-temporal hint (data used once)
__device__ __forceinline__ void buf_lds16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                             void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t)lds_dst, 16, voff, soff, 0, 2);
}

}  // namespace bfp8
