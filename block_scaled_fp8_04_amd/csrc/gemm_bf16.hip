// gemm_bf16.hip - the BF16 branch of linear() on gfx950: C = A * B^T with bf16
// A [M, K] (activations) and bf16 B [N, K] (a weight expanded by
// weight_dequant), fp32 accumulation, bf16 output (pyshine "DeepSeek-V3"
// tour, "FP8 with per-block scales": the weight is dequantized and multiplied
// by an ordinary BF16 matmul).
//
// Design (wave64, v_mfma_f32_16x16x32_bf16):
//  * The K loop walks steps of 64 elements: one step of a row is 128 bytes,
//    the same LDS row format as the fp8 kernel (eight 16-byte chunks, chunk c
//    of row r stored at c ^ swz(r), conflict-free for the fragment reads).
//    A step feeds two MFMAs per 16x16 sub-tile (K 0-31 and 32-63).
//  * Lane l supplies row l & 15 of a sub-tile and the 8 consecutive K elements
//    8 (l >> 4) .. +8 of a 32-wide half: one 16-byte LDS read per fragment.
//    A and B use the same pattern, so the K order inside the MFMA cannot
//    change the sum.  The MFMA accumulates straight into the fp32 sum (no
//    block scales on this branch).
//  * Operands go weight-first, so a lane owns one output row and four
//    consecutive columns of each sub-tile, as in the fp8 kernel; interior
//    tiles of the two larger shapes store them through LDS as whole 128-byte
//    row pieces, other tiles directly (8 bytes per lane and sub-tile).
//  * Tiles 256x256 (8 waves of 128x64, 2 LDS stages of 64 KB), 256x128
//    (8 waves of 64x64, 3 stages of 48 KB) and 64x64 (4 waves of 32x32,
//    3 stages of 16 KB) by problem size.  A and B steps go straight to LDS
//    with buffer loads; the stages are distinct __shared__ arrays and the
//    K loop is unrolled by the stage count (precise LDS waits, as in the fp8
//    kernel); a vmcnt-counted wait and one barrier open each step.
//  * Rows past M and columns past N read a clamped valid row and are never
//    stored; sub-tile rows entirely past M skip their MFMAs.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kStep = 64;           // K elements per LDS stage
constexpr int kRowBytes = 128;      // bytes of one row per stage

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const int num = (int)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num, 0x00020000);
}

template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_>
struct BfTile {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NSTAGE = NSTAGE_;
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // As in the fp8 GEMM: in the two-stage eight-wave tile waves 0..3 issue
    // every A and B load and waves 4..7 (one priority level up) only multiply
    // (3% faster on 8192 x 18432 x 7168).
    static constexpr int LOADERS = (NSTAGE == 2 && WAVES == 8) ? 4 : WAVES;
    static constexpr int A_INSTR = BM / 8 / LOADERS, B_INSTR = BN / 8 / LOADERS;
    static constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR;
    static_assert(BM % (8 * LOADERS) == 0 && BN % (8 * LOADERS) == 0,
                  "tile rows must split over the loading waves");
    static_assert(TM >= 1 && TN >= 1, "a wave holds at least one sub-tile");
    static_assert(NSTAGE >= 2 && NSTAGE <= 3 && NSTAGE * STAGE <= 158 * 1024, "stages must fit in LDS");
};

template <class T>
struct BfStages {
    uint8_t* p[3];
};
template <int S>
struct BfStageId {
    static constexpr int value = S;
};

// Where a tile's sums go when it runs only K steps [ks_lo, ks_hi) of the
// split last round: fp32 row r, column n at ws[r * ldw + n - n_base].
struct BfPartial {
    int64_t ks_lo = 0, ks_hi = -1;      // ks_hi < 0: all K steps, bf16 output
    float* ws = nullptr;
    int64_t ldw = 0, n_base = 0;
};

template <class T, bool kGuard, bool kPartial = false>
__device__ __forceinline__ void bf16_tile(const uint16_t* __restrict__ a,
                                          const uint16_t* __restrict__ b,
                                          uint16_t* __restrict__ c, int64_t m0, int64_t M,
                                          int64_t n0, int64_t N, int64_t K,
                                          const BfStages<T>& st, BfPartial part = BfPartial{}) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / T::WAVES_N) * T::WM;
    const int wn0 = (wave % T::WAVES_N) * T::WN;
    // the K steps this tile multiplies: [KS0, KS)
    const int64_t KS0 = part.ks_lo, KS = part.ks_hi < 0 ? K / kStep : part.ks_hi;
    const int64_t rows_a = (M - m0) < T::BM ? (M - m0) : T::BM;
    const int64_t rows_b = (N - n0) < T::BN ? (N - n0) : T::BN;
    const int64_t row_bytes = 2 * K;

    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a + m0 * K, (uint64_t)rows_a * row_bytes);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(b + n0 * K, (uint64_t)rows_b * row_bytes);

    const int lrow = lane >> 3;
    uint32_t a_off[T::A_INSTR], b_off[T::B_INSTR];
#pragma unroll
    for (int i = 0; i < T::A_INSTR; ++i) {
        int row = (wave * T::A_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        row = row < rows_a ? row : (int)rows_a - 1;
        a_off[i] = (uint32_t)(row * row_bytes) + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < T::B_INSTR; ++i) {
        int row = (wave * T::B_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        row = row < rows_b ? row : (int)rows_b - 1;
        b_off[i] = (uint32_t)(row * row_bytes) + chunk * 16;
    }
    auto issue = [&](int64_t ks, uint8_t* base) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)(ks * kRowBytes);
        if (T::LOADERS < T::WAVES && wave >= T::LOADERS) return;
#pragma unroll
        for (int i = 0; i < T::A_INSTR; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_a, (lds_ptr_t)(base + (wave * T::A_INSTR + i) * 1024), 16, a_off[i], ko, 0, 0);
#pragma unroll
        for (int i = 0; i < T::B_INSTR; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs_b, (lds_ptr_t)(base + T::A_BYTES + (wave * T::B_INSTR + i) * 1024), 16, b_off[i],
                ko, 0, 0);
    };

    if (T::WAVES == 8 && wave >= 4) __builtin_amdgcn_s_setprio(1);
    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    int tm_valid = T::TM;
    if (kGuard) {
        const int64_t rows = M - (m0 + wm0);
        tm_valid = rows <= 0 ? 0 : (rows >= 16 * T::TM ? T::TM : (int)((rows + 15) / 16));
        tm_valid = __builtin_amdgcn_readfirstlane(tm_valid);
    }

    issue(KS0, st.p[0]);
    if (T::NSTAGE > 2 && KS0 + 1 < KS) issue(KS0 + 1, st.p[1]);

    const int lr = lane & 15;
    const int g = lane >> 4;
    // fragment half h of row r: logical chunk 4 h + g
    const int off_h0 = ((g ^ swz(lr)) << 4);
    const int off_h1 = (((4 + g) ^ swz(lr)) << 4);

    auto frag = [&](const uint8_t* row_base, int off) __attribute__((always_inline)) {
        return __builtin_bit_cast(v8bf, *(const uint4*)(row_base + off));
    };

    auto step = [&](int64_t ks, auto S_) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        constexpr int SF = (S + T::NSTAGE - 1) % T::NSTAGE;
        if (ks + T::NSTAGE - 2 < KS)
            wait_vmcnt<T::LOADS_PER_STAGE * (T::NSTAGE - 2)>();
        else
            wait_vmcnt<0>();
        barrier_lds();
        if (ks + T::NSTAGE - 1 < KS) issue(ks + T::NSTAGE - 1, st.p[SF]);

        const uint8_t* As = st.p[S];
        const uint8_t* Bs = As + T::A_BYTES;
        v8bf fb0[T::TN], fb1[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const uint8_t* q = Bs + (wn0 + 16 * j + lr) * kRowBytes;
            fb0[j] = frag(q, off_h0);
            fb1[j] = frag(q, off_h1);
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            if (!kGuard || i < tm_valid) {
                const uint8_t* r = As + (wm0 + 16 * i + lr) * kRowBytes;
                const v8bf fa0 = frag(r, off_h0);
                const v8bf fa1 = frag(r, off_h1);
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb0[j], fa0, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb1[j], fa1, acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    for (int64_t ks0 = KS0; ks0 < KS; ks0 += T::NSTAGE) {
        step(ks0, BfStageId<0>{});
        if (ks0 + 1 < KS) step(ks0 + 1, BfStageId<1>{});
        if constexpr (T::NSTAGE > 2) {
            if (ks0 + 2 < KS) step(ks0 + 2, BfStageId<2>{});
        }
    }

    // epilogue: lane holds row m0 + wm0 + 16 i + lr, columns n0 + wn0 + 16 j + 4 g + 0..3
    if constexpr (kPartial) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int64_t row = m0 + wm0 + 16 * i + lr;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int64_t col = n0 + wn0 + 16 * j + 4 * g;
                if (row < M && col + 3 < N)
                    *(v4f*)(part.ws + row * part.ldw + (col - part.n_base)) = acc[i][j];
            }
        }
        return;
    }
    const bool interior = (m0 + T::BM <= M) && (n0 + T::BN <= N);
    const bool vec = interior && (N % 4 == 0) && (((uintptr_t)c & 7u) == 0);
    // Staged store (as in the fp8 GEMM): after a barrier (no loads are in
    // flight after the last K step) the first stage is free; each wave turns
    // kRP of its rows at a time into bf16 rows of 128 bytes there (16-byte
    // chunks XOR-swizzled by row) and stores whole 128-byte row pieces, 16
    // bytes per lane, instead of 8 bytes per lane and sub-tile.
    constexpr int kRP = T::WAVES * 64 * 128 <= T::STAGE ? 64 : 32;
    constexpr int kSub = kRP / 16;
    if constexpr (T::WN == 64 && T::TM % kSub == 0 && T::WAVES * kRP * 128 <= T::STAGE) {
        if (vec && (N % 8 == 0) && (((uintptr_t)c & 15u) == 0)) {
            __syncthreads();                      // every wave is past its last LDS read
            uint8_t* buf = st.p[0] + wave * (kRP * 128);
#pragma unroll
            for (int h = 0; h < T::TM / kSub; ++h) {
#pragma unroll
                for (int i = 0; i < kSub; ++i) {
                    const int r = 16 * i + lr;
#pragma unroll
                    for (int j = 0; j < T::TN; ++j) {
                        const int byte = (16 * j + 4 * g) * 2;
                        uint2 v;
                        v.x = pack_bf16x2(acc[kSub * h + i][j][0], acc[kSub * h + i][j][1]);
                        v.y = pack_bf16x2(acc[kSub * h + i][j][2], acc[kSub * h + i][j][3]);
                        *(uint2*)(buf + r * 128 + (((byte >> 4) ^ (r & 7)) << 4) + (byte & 15)) = v;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                uint4 o[kRP / 8];
#pragma unroll
                for (int q = 0; q < kRP / 8; ++q) {
                    const int r = 8 * q + (lane >> 3), ch = lane & 7;
                    o[q] = *(const uint4*)(buf + r * 128 + ((ch ^ (r & 7)) << 4));
                }
#pragma unroll
                for (int q = 0; q < kRP / 8; ++q) {
                    const int r = 8 * q + (lane >> 3), ch = lane & 7;
                    *(uint4*)(c + (m0 + wm0 + kRP * h + r) * N + n0 + wn0 + ch * 8) = o[q];
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
            return;
        }
    }
    if (vec) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            uint16_t* crow = c + (m0 + wm0 + 16 * i + lr) * N + n0 + wn0 + 4 * g;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                uint2 v;
                v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(uint2*)(crow + 16 * j) = v;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int64_t row = m0 + wm0 + 16 * i + lr;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t col = n0 + wn0 + 16 * j + 4 * g + r;
                    if (row < M && col < N) c[row * N + col] = (uint16_t)bf16_rne_bits(acc[i][j][r]);
                }
            }
        }
    }
}

// Workgroup id -> tile, XCD-aware: ids are regrouped XCD by XCD (they are
// dealt round-robin over the 8 XCDs), then walked in bands of 4 M-tiles with
// M fastest, so one XCD's resident workgroups share A and B slices in L2.
__device__ __forceinline__ void bf16_tile_of(int id, int nwg, int mt, int nt, int& tm, int& tn) {
    constexpr int XCDS = 8, GM = 4;
    const int xcd = id % XCDS, local = id / XCDS;
    const int per = nwg / XCDS, rem = nwg % XCDS;
    const int lin = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int band = lin / (GM * nt);
    const int first_m = band * GM;
    const int rows_in_band = (mt - first_m) < GM ? (mt - first_m) : GM;
    const int in_band = lin - band * GM * nt;
    tm = first_m + in_band % rows_in_band;
    tn = in_band / rows_in_band;
}

template <class T>
__global__ __launch_bounds__(T::THREADS, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ a,
                                                                  const uint16_t* __restrict__ b,
                                                                  uint16_t* __restrict__ c,
                                                                  int64_t M, int64_t N, int64_t K,
                                                                  int mt, int nt) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[T::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[T::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[T::NSTAGE > 2 ? T::STAGE : 16];
    const BfStages<T> st = {{st0, st1, st2}};
    int tm, tn;
    bf16_tile_of(blockIdx.x, gridDim.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM;
    if (m0 + T::BM <= M)
        bf16_tile<T, false>(a, b, c, m0, M, (int64_t)tn * T::BN, N, K, st);
    else
        bf16_tile<T, true>(a, b, c, m0, M, (int64_t)tn * T::BN, N, K, st);
}

// The split last round's tail columns: tile t of split s (blockIdx = s * tiles
// + t) multiplies K steps [s * ks_per, (s + 1) * ks_per) of tile t of the
// columns from n1 and writes fp32 sums to ws[s][M][N - n1].
template <class T>
__global__ __launch_bounds__(T::THREADS, 1) void gemm_bf16_tail_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, float* __restrict__ ws,
    int64_t M, int64_t N, int64_t K, int mt, int nt_tail, int64_t n1, int64_t ks_per) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[T::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[T::STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[T::NSTAGE > 2 ? T::STAGE : 16];
    const BfStages<T> st = {{st0, st1, st2}};
    const int tiles = mt * nt_tail;
    const int split = blockIdx.x / tiles;
    int tm, tn;
    bf16_tile_of(blockIdx.x - split * tiles, tiles, mt, nt_tail, tm, tn);
    const int64_t KS = K / kStep;
    BfPartial part;
    part.ks_lo = split * ks_per;
    part.ks_hi = part.ks_lo + ks_per < KS ? part.ks_lo + ks_per : KS;
    part.ldw = N - n1;
    part.ws = ws + (int64_t)split * M * part.ldw;
    part.n_base = n1;
    bf16_tile<T, false, true>(a, b, nullptr, (int64_t)tm * T::BM, M, n1 + (int64_t)tn * T::BN, N,
                              K, st, part);
}

using BfSquare = BfTile<256, 256, 2, 4, 2>;
using BfWide = BfTile<256, 128, 4, 2, 3>;
using BfSmall = BfTile<64, 64, 2, 2, 3>;

template <class T>
hipError_t launch_bf16(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream) {
    const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
    hipLaunchKernelGGL(gemm_bf16_kernel<T>, dim3(mt * nt), dim3(T::THREADS), 0, stream,
                       (const uint16_t*)a, (const uint16_t*)b, (uint16_t*)c, M, N, K, mt, nt);
    return hipGetLastError();
}

}  // namespace

const char* gemm_bf16_config_name(int64_t M, int64_t N, int64_t K) {
    (void)K;
    const int64_t cus = device_cu_count();
    // 256 x 256 from 5/8 of a tile per CU up (measured 20-22% faster than 256 x 128 at
    // 256-448 tiles), as for the fp8 GEMM
    if (M > 128 && ((M + 255) / 256) * ((N + 255) / 256) >= cus * 5 / 8) return "bf16 256x256, 8 waves of 128x64";
    if (M > 128 && ((M + 255) / 256) * ((N + 127) / 128) >= cus / 2) return "bf16 256x128, 8 waves of 64x64";
    return "bf16 64x64, 4 waves of 32x32";
}

hipError_t launch_gemm_bf16(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const int64_t cus = device_cu_count();
    // with a workspace, the split last round of the fp8 GEMM (tail_plan); its plan takes
    // the 256 x 256 tile, which this shape then uses too (at least 256 tiles)
    const TailPlan tp = tail_plan(M, N, K);
    if (workspace && tp.splits > 0 && workspace_bytes >= tail_workspace_bytes(M, N, K) &&
        ((uintptr_t)c & 7u) == 0) {
        const int mt = (int)(M / 256);
        const int64_t n1 = (int64_t)tp.nt_main * 256;
        hipLaunchKernelGGL(gemm_bf16_kernel<BfSquare>, dim3(mt * tp.nt_main),
                           dim3(BfSquare::THREADS), 0, stream, (const uint16_t*)a,
                           (const uint16_t*)b, (uint16_t*)c, M, N, K, mt, tp.nt_main);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // the K steps of 64 shared out over the splits (K need only be a multiple of 64)
        const int64_t ks = K / kStep, ks_per = (ks + tp.splits - 1) / tp.splits;
        hipLaunchKernelGGL(gemm_bf16_tail_kernel<BfSquare>, dim3(mt * tp.nt_tail * tp.splits),
                           dim3(BfSquare::THREADS), 0, stream, (const uint16_t*)a,
                           (const uint16_t*)b, (float*)workspace, M, N, K, mt, tp.nt_tail, n1,
                           ks_per);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_tail_reduce((const float*)workspace, c, M, N, n1, tp.splits, stream);
    }
    // 256 x 256 from 5/8 of a tile per CU up (measured 20-22% faster than 256 x 128 at
    // 256-448 tiles), as for the fp8 GEMM
    if (M > 128 && ((M + 255) / 256) * ((N + 255) / 256) >= cus * 5 / 8)
        return launch_bf16<BfSquare>(a, b, c, M, N, K, stream);
    if (M > 128 && ((M + 255) / 256) * ((N + 127) / 128) >= cus / 2)
        return launch_bf16<BfWide>(a, b, c, M, N, K, stream);
    return launch_bf16<BfSmall>(a, b, c, M, N, K, stream);
}

}  // namespace bfp8
