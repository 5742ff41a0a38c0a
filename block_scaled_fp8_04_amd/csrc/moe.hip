// moe.hip - MoE dispatch and combine on gfx950, either side of the grouped GEMM.
//
// The routed-expert step of DeepSeek-V3 counts the tokens of every expert,
// and for each local expert with tokens selects those tokens in ascending
// order, runs the expert on them and adds the expert's output, times the
// routing weight, into a zero-initialised y ("Behavior traces -
// deepseek-ai/DeepSeek-V3", MoE trace; a GPU holds a contiguous range of
// experts, "Data flow", expert sharding).  On the device this is:
//
//   dispatch: a stable counting sort of the flat (token, slot) list by local
//     expert id.  Rows of expert g are offsets[g] .. offsets[g+1]; inside an
//     expert, rows follow (token, slot) order, so tokens ascend.
//     1. dispatch_rank_kernel: workgroup b owns entries 256b .. 256b+255 (one
//        per thread).  Inside each wave, lanes with the same expert are found
//        by a ballot loop (one pass per distinct expert in the wave), which
//        gives each entry its rank among earlier lanes of that expert; the
//        four waves' counts go through LDS to make the rank block-wide.  The
//        entry's (expert, rank in block) is parked in slot_row, and the
//        block's count of every expert goes to ws[g * B + b].
//     2. dispatch_scan_kernel: one workgroup runs an exclusive scan over ws
//        in (expert, block) order.  That is exactly the first row of every
//        (expert, block) pair; offsets[g] is the value at (g, 0).
//     3. dispatch_place_kernel: row = ws[g * B + b] + rank; writes slot_row
//        and row_token.
//     When the count table is small (it fits 64 KB of LDS, and its size times
//     the number of workgroups is at most kFusedScanReads), steps 2 and 3 are
//     one kernel instead, dispatch_scan_place_kernel: every workgroup copies
//     the table into LDS and sums it itself (per expert the count over all
//     blocks and over the blocks before its own, then an exclusive scan over
//     experts), which gives the same row for every entry without a
//     single-workgroup pass between rank and place.
//   combine: y[t, :] = bf16( sum over the token's local slots, in slot
//     order, of weight * out[slot_row] ) accumulated in fp32.  One workgroup
//     per (token, 2048-column chunk), tokens along grid x; a lane owns 8
//     columns (16-byte loads of every gathered row, one 16-byte store).
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

constexpr int kDispatchBlock = 256;          // entries per workgroup of the rank/place kernels
constexpr int kDispatchWaves = kDispatchBlock / 64;

// rank of entry (expert e, rank r in its block) parked in slot_row between kernels
__device__ __forceinline__ int32_t park(int e, int r) { return (e << 16) | r; }

__global__ __launch_bounds__(kDispatchBlock) void dispatch_rank_kernel(
    const int32_t* __restrict__ topk, int64_t n, int32_t lo, int G, int nblk,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ ws) {
    __shared__ int32_t wcnt[kDispatchWaves][kMoeMaxGroups];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kDispatchWaves * G; i += kDispatchBlock) wcnt[i / G][i % G] = 0;
    __syncthreads();

    const int64_t i = (int64_t)blockIdx.x * kDispatchBlock + tid;
    int e = -1;
    if (i < n) {
        const int64_t d = (int64_t)topk[i] - lo;
        e = (d >= 0 && d < G) ? (int)d : -1;
    }
    // ballot loop: one pass per distinct local expert present in this wave
    int rank = 0;
    uint64_t active = __ballot(e >= 0);
    while (active) {
        const int leader = __ffsll((unsigned long long)active) - 1;
        const int el = __builtin_amdgcn_readlane(e, leader);
        const uint64_t m = __ballot(e == el);
        if (e == el) rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == leader) wcnt[wave][el] = __popcll(m);
        active &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
        for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
        slot_row[i] = park(e, rank);
    } else if (i < n) {
        slot_row[i] = -1;
    }
    for (int g = tid; g < G; g += kDispatchBlock) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kDispatchWaves; ++w) c += wcnt[w][g];
        ws[(int64_t)g * nblk + blockIdx.x] = c;
    }
}

// Exclusive scan of ws[0 .. G*nblk) in place by one workgroup of 1024
// threads, 4096 elements per step with a running carry.  off[g] = the scanned
// value at (g, 0); off[G] = the total.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ ws, int G,
                                                             int nblk, int32_t* __restrict__ off) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t wpre[17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t len = (int64_t)G * nblk;
    if (nblk == 0)
        for (int g = tid; g < G; g += 1024) off[g] = 0;
    int32_t carry = 0;
    for (int64_t base = 0; base < len; base += 4096) {
        int32_t v[4];
        const int64_t j0 = base + (int64_t)tid * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (j0 + q < len) ? ws[j0 + q] : 0;
        const int32_t s = v[0] + v[1] + v[2] + v[3];
        int32_t incl = s;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int32_t y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        if (tid == 0) {
            int32_t run = 0;
            for (int w = 0; w < 16; ++w) {
                wpre[w] = run;
                run += wsum[w];
            }
            wpre[16] = run;
        }
        __syncthreads();
        int32_t x = carry + wpre[wave] + incl - s;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t j = j0 + q;
            if (j < len) {
                ws[j] = x;
                if (j % nblk == 0) off[j / nblk] = x;
            }
            x += v[q];
        }
        carry += wpre[16];
        __syncthreads();            // wsum / wpre are rewritten by the next step
    }
    if (tid == 0) off[G] = carry;
}

__global__ __launch_bounds__(kDispatchBlock) void dispatch_place_kernel(
    int64_t n, int k, int nblk, const int32_t* __restrict__ ws, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token) {
    const int64_t i = (int64_t)blockIdx.x * kDispatchBlock + threadIdx.x;
    if (i >= n) return;
    const int32_t v = slot_row[i];
    if (v < 0) return;
    const int e = v >> 16, r = v & 0xFFFF;
    const int32_t row = ws[(int64_t)e * nblk + blockIdx.x] + r;
    slot_row[i] = row;
    row_token[row] = (int32_t)(i / k);
}

// Limits of the fused kernel: the count table fits its LDS, and the table
// entries read by all its workgroups together stay bounded.
constexpr int kFusedScanLds = 16384;                      // int32 entries (64 KB)
constexpr int64_t kFusedScanReads = int64_t(1) << 22;

// Steps 2 and 3 in one kernel (workgroup b = the rank kernel's workgroup b).
// The workgroup copies the count table into LDS (all loads in flight at
// once), then base[g] = (entries of experts before g) + (entries of expert g
// in blocks before b), which is ws[g * nblk + b] after step 2's exclusive scan.
__global__ __launch_bounds__(kDispatchBlock) void dispatch_scan_place_kernel(
    int64_t n, int k, int G, int nblk, const int32_t* __restrict__ ws,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token, int32_t* __restrict__ off) {
    extern __shared__ int32_t tab[];                      // [G][nblk]
    __shared__ int32_t tot[kMoeMaxGroups];
    __shared__ int32_t base[kMoeMaxGroups];
    constexpr int U = 32;                                 // loads per thread in flight
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int64_t i = (int64_t)b * kDispatchBlock + tid;
    const int32_t parked = i < n ? slot_row[i] : -1;
    const int len = G * nblk;
    for (int q0 = 0; q0 < len; q0 += U * kDispatchBlock) {
        int32_t x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * kDispatchBlock + tid;
            x[u] = q < len ? ws[q] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * kDispatchBlock + tid;
            if (q < len) tab[q] = x[u];
        }
    }
    __syncthreads();
    // tpr lanes (a power of two, inside one wave) sum one expert's row
    int tpr = 64;
    while (tpr > 1 && tpr * G > kDispatchBlock) tpr >>= 1;
    const int rows_per_pass = kDispatchBlock / tpr;
    const int sub = lane & (tpr - 1);
    for (int g0 = 0; g0 < G; g0 += rows_per_pass) {
        const int g = g0 + tid / tpr;
        int32_t t = 0, below = 0;
        if (g < G) {
            const int32_t* row = tab + g * nblk;
#pragma unroll 8
            for (int j = sub; j < nblk; j += tpr) {
                const int32_t v = row[j];
                t += v;
                below += j < b ? v : 0;
            }
        }
        for (int d = 1; d < tpr; d <<= 1) {
            t += __shfl_xor(t, d);
            below += __shfl_xor(below, d);
        }
        if (g < G && sub == 0) {
            tot[g] = t;
            base[g] = below;
        }
    }
    __syncthreads();
    if (wave == 0) {
        int32_t carry = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            const int32_t v = g < G ? tot[g] : 0;
            int32_t incl = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int32_t y = __shfl_up(incl, d);
                if (lane >= d) incl += y;
            }
            if (g < G) {
                const int32_t excl = carry + incl - v;
                base[g] += excl;
                if (b == 0) off[g] = excl;
            }
            carry += __shfl(incl, 63);
        }
        if (b == 0 && lane == 0) off[G] = carry;
    }
    __syncthreads();
    if (parked < 0) return;
    const int e = parked >> 16, r = parked & 0xFFFF;
    const int32_t row = base[e] + r;
    slot_row[i] = row;
    row_token[row] = (int32_t)(i / k);
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t k, int32_t G) {
    const int64_t n = T * (int64_t)k;
    const int64_t nblk = (n + kDispatchBlock - 1) / kDispatchBlock;
    return (size_t)(nblk * (int64_t)G * 4 + 15) / 16 * 16;
}

hipError_t launch_moe_dispatch(const int32_t* topk, int64_t T, int32_t k, int32_t lo, int32_t G,
                               int32_t* off, int32_t* row_token, int32_t* slot_row, void* ws,
                               hipStream_t stream) {
    const int64_t n = T * (int64_t)k;
    const int nblk = (int)((n + kDispatchBlock - 1) / kDispatchBlock);
    int32_t* w = (int32_t*)ws;
    if (nblk > 0) {
        hipLaunchKernelGGL(dispatch_rank_kernel, dim3(nblk), dim3(kDispatchBlock), 0, stream, topk,
                           n, lo, (int)G, nblk, slot_row, w);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t len = (int64_t)G * nblk;
        if (len <= kFusedScanLds && len * nblk <= kFusedScanReads) {
            hipLaunchKernelGGL(dispatch_scan_place_kernel, dim3(nblk), dim3(kDispatchBlock),
                               (size_t)len * 4, stream, n, (int)k, (int)G, nblk, w, slot_row,
                               row_token, off);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, stream, w, (int)G, nblk, off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nblk == 0) return e;
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(nblk), dim3(kDispatchBlock), 0, stream, n,
                       (int)k, nblk, w, slot_row, row_token);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine

constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 8;   // columns per workgroup

// Vector path: N % 8 == 0, out and y 16-byte aligned.  Block (x = chunk,
// y = token); lane owns columns c .. c+7.
__global__ __launch_bounds__(kCombineThreads) void combine_vec_kernel(
    const uint16_t* __restrict__ out, int64_t rows_cap, const int32_t* __restrict__ slot_row,
    const float* __restrict__ weight, uint16_t* __restrict__ y, int k, int64_t N) {
    const int64_t t = blockIdx.x;
    const int64_t c = (int64_t)blockIdx.y * kCombineCols + (int64_t)threadIdx.x * 8;
    if (c >= N) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int32_t r = slot_row[t * k + j];
        if (r < 0 || r >= rows_cap) continue;
        const float w = weight[t * k + j];
        const uint4 v = load_nt(reinterpret_cast<const uint4*>(out + (int64_t)r * N + c));
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] = __builtin_fmaf(w, bf16_lo(p[q]), acc[2 * q]);
            acc[2 * q + 1] = __builtin_fmaf(w, bf16_hi(p[q]), acc[2 * q + 1]);
        }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    store_nt(reinterpret_cast<uint4*>(y + t * N + c), o);
}

// Any N and 2-byte alignment: one column per lane.
__global__ __launch_bounds__(kCombineThreads) void combine_scalar_kernel(
    const uint16_t* __restrict__ out, int64_t rows_cap, const int32_t* __restrict__ slot_row,
    const float* __restrict__ weight, uint16_t* __restrict__ y, int k, int64_t N) {
    const int64_t t = blockIdx.x;
    const int64_t c = (int64_t)blockIdx.y * kCombineThreads + threadIdx.x;
    if (c >= N) return;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
        const int32_t r = slot_row[t * k + j];
        if (r < 0 || r >= rows_cap) continue;
        acc = __builtin_fmaf(weight[t * k + j], bf16_lo(out[(int64_t)r * N + c]), acc);
    }
    y[t * N + c] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
}

hipError_t launch_moe_combine(const void* out, int64_t rows_cap, const int32_t* slot_row,
                              const float* weight, void* y, int64_t T, int32_t k, int64_t N,
                              hipStream_t stream) {
    const bool vec = (N % 8 == 0) && ((uintptr_t)out % 16 == 0) && ((uintptr_t)y % 16 == 0);
    if (vec) {
        const dim3 grid((unsigned)T, (unsigned)((N + kCombineCols - 1) / kCombineCols));
        hipLaunchKernelGGL(combine_vec_kernel, grid, dim3(kCombineThreads), 0, stream,
                           (const uint16_t*)out, rows_cap, slot_row, weight, (uint16_t*)y, (int)k,
                           N);
    } else {
        const dim3 grid((unsigned)T, (unsigned)((N + kCombineThreads - 1) / kCombineThreads));
        hipLaunchKernelGGL(combine_scalar_kernel, grid, dim3(kCombineThreads), 0, stream,
                           (const uint16_t*)out, rows_cap, slot_row, weight, (uint16_t*)y, (int)k,
                           N);
    }
    return hipGetLastError();
}

}  // namespace bfp8
