// gemm.hip - block-scaled fp8 GEMM (plain and grouped) on gfx950.
//
// c[m, n] = bf16( sum_kb P_kb[m, n] * a_s[m, kb] * b_s[n/128, kb] ),
// P_kb[m, n] = sum_{k in block kb} a[m, k] * b[n, k]
// ("Data flow - deepseek-ai/DeepSeek-V3", FP8 quantization bullet: fp8_gemm
// multiplies scaled blocks and accumulates in fp32; pyshine tour, "FP8 with
// per-block scales").  a is [M, K] and b is a Linear weight [N, K], both
// K-contiguous, so C = A * B^T.
//
// Design (gfx950, wave64):
//  * One 128-wide K block is exactly the K extent of one
//    v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3 -> fp32).  Each 16x16 sub-tile
//    of a wave's output gets one MFMA per K block into a zeroed accumulator,
//    and that block product is folded into the running fp32 sum with one FMA
//    per element: acc += P * (a_s[row] * b_s).  The weight-scale block is the
//    same for all of a wave's columns (a wave's N range lies inside one
//    128-column block), so the fold needs one scale per row.
//  * A workgroup is 4 waves in a 2 x 2 layout over a BM x BN tile.  A and B
//    tiles of one K block (BM x 128 and BN x 128 bytes) are staged through LDS,
//    double buffered: while the waves multiply stage s, the next K block's
//    global loads are in flight in registers and are written to stage s^1.
//    One barrier per K block.
//  * LDS rows are 128 bytes; the eight 16-byte chunks of row r are stored at
//    chunk position (chunk ^ swz(r)) (see swz below), so the 16 rows read
//    together by a fragment load (same logical chunk) hit no bank twice.
//  * MFMA operand layout: lane l supplies row (l & 15) of the sub-tile and the
//    32 K-bytes starting at 32 * (l >> 4), for A and B alike, so each K index
//    pairs the same position of A and B.  The accumulator layout of a 16x16
//    fp32 result is: lane l holds column (l & 15), rows 4*(l >> 4) + 0..3.
//  * Rows past M (or past a group's end) and columns past N read a clamped,
//    valid row and are never stored.
#include "device_codec.hpp"
#include "internal.hpp"

namespace bfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int BM_, int BN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WM = BM / 2, WN = BN / 2;      // per-wave extent (2 x 2 waves)
    static constexpr int TM = WM / 16, TN = WN / 16;    // 16 x 16 sub-tiles per wave
    static constexpr int A_BYTES = BM * kBlock;
    static constexpr int B_BYTES = BN * kBlock;
    static constexpr int A_LOADS = A_BYTES / (256 * 16);
    static constexpr int B_LOADS = B_BYTES / (256 * 16);
    static constexpr int STAGE = A_BYTES + B_BYTES + BM * 4;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for 256 threads");
    static_assert(TM >= 1 && TN >= 1, "wave tile must hold a 16x16 sub-tile");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one scale block");
};

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

// Computes rows [m0, min(m0 + BM, m_end)) x columns [n0, min(n0 + BN, N)) of c.
template <class T>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a,
                                          const float* __restrict__ as,
                                          const uint8_t* __restrict__ b,
                                          const float* __restrict__ bs,
                                          uint16_t* __restrict__ c, int64_t m0, int64_t m_end,
                                          int64_t n0, int64_t N, int64_t K, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave >> 1) * T::WM;
    const int wn0 = (wave & 1) * T::WN;
    const int64_t KB = K / kBlock;
    const int64_t NB = (N + kBlock - 1) / kBlock;

    // global sources and LDS destinations of this thread's 16-byte chunks
    const uint8_t* a_src[T::A_LOADS];
    const uint8_t* b_src[T::B_LOADS];
    int a_dst[T::A_LOADS], b_dst[T::B_LOADS];
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
        const int ch = tid + 256 * i, row = ch >> 3, col = ch & 7;
        int64_t grow = m0 + row;
        grow = grow < m_end ? grow : m_end - 1;
        a_src[i] = a + grow * K + col * 16;
        a_dst[i] = row * kBlock + ((col ^ swz(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) {
        const int ch = tid + 256 * i, row = ch >> 3, col = ch & 7;
        int64_t gcol = n0 + row;
        gcol = gcol < N ? gcol : N - 1;
        b_src[i] = b + gcol * K + col * 16;
        b_dst[i] = T::A_BYTES + row * kBlock + ((col ^ swz(row)) << 4);
    }
    const float* sa_src = nullptr;
    if (tid < T::BM) {
        int64_t grow = m0 + tid;
        grow = grow < m_end ? grow : m_end - 1;
        sa_src = as + grow * KB;
    }
    int64_t nblk = (n0 + wn0) >> 7;
    nblk = nblk < NB ? nblk : NB - 1;
    const float* sb_src = bs + nblk * KB;

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 ra[T::A_LOADS], rb[T::B_LOADS];
    float rsa = 0.f;

    auto load_regs = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < T::A_LOADS; ++i) ra[i] = *(const uint4*)(a_src[i] + kb * kBlock);
#pragma unroll
        for (int i = 0; i < T::B_LOADS; ++i) rb[i] = *(const uint4*)(b_src[i] + kb * kBlock);
        if (tid < T::BM) rsa = sa_src[kb];
    };
    auto store_lds = [&](int stage) {
        uint8_t* base = lds + stage * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::A_LOADS; ++i) *(uint4*)(base + a_dst[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < T::B_LOADS; ++i) *(uint4*)(base + b_dst[i]) = rb[i];
        if (tid < T::BM) ((float*)(base + T::A_BYTES + T::B_BYTES))[tid] = rsa;
    };

    load_regs(0);
    store_lds(0);
    __syncthreads();

    const int lr = lane & 15;
    const int lk = (lane >> 4) * 2;               // first of this lane's two 16-byte chunks
    const int off0 = ((lk ^ swz(lr)) << 4);
    const int off1 = (((lk + 1) ^ swz(lr)) << 4);
    const int srow = 4 * (lane >> 4);

    for (int64_t kb = 0; kb < KB; ++kb) {
        const int cur = (int)(kb & 1);
        const bool more = kb + 1 < KB;
        if (more) load_regs(kb + 1);

        const uint8_t* As = lds + cur * T::STAGE;
        const uint8_t* Bs = As + T::A_BYTES;
        const float* Ss = (const float*)(Bs + T::B_BYTES);
        v8i fa[T::TM], fb[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const uint8_t* r = As + (wm0 + 16 * i + lr) * kBlock;
            fa[i] = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const uint8_t* r = Bs + (wn0 + 16 * j + lr) * kBlock;
            fb[j] = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
        }
        const float sbv = sb_src[kb];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const v4f sa4 = *(const v4f*)(Ss + wm0 + 16 * i + srow);
            const v4f sc = sa4 * sbv;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fa[i], fb[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                acc[i][j] = p * sc + acc[i][j];
            }
        }
        if (more) store_lds(cur ^ 1);
        __syncthreads();
    }

    // epilogue: fp32 -> bf16 (nearest even), masked to the valid rows / columns
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int64_t col = n0 + wn0 + 16 * j + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm0 + 16 * i + srow + r;
                if (row < m_end && col < N) c[row * N + col] = (uint16_t)bf16_rne_bits(acc[i][j][r]);
            }
        }
    }
}

template <class T>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint8_t* __restrict__ a,
                                                      const float* __restrict__ as,
                                                      const uint8_t* __restrict__ b,
                                                      const float* __restrict__ bs,
                                                      uint16_t* __restrict__ c, int64_t M,
                                                      int64_t N, int64_t K, int mt, int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * T::STAGE];
    // bands of 8 M-tiles: within a band, consecutive workgroups walk down the
    // band's M-tiles for one N-tile, then move to the next N-tile.
    constexpr int GM = 8;
    const int id = blockIdx.x;
    const int band = id / (GM * nt);
    const int first_m = band * GM;
    const int rows_in_band = (mt - first_m) < GM ? (mt - first_m) : GM;
    const int in_band = id - band * GM * nt;
    const int tm = first_m + in_band % rows_in_band;
    const int tn = in_band / rows_in_band;
    gemm_tile<T>(a, as, b, bs, c, (int64_t)tm * T::BM, M, (int64_t)tn * T::BN, N, K, lds);
}

// Persistent grouped kernel: workgroups stride over the tiles of all groups.
// Group g owns ceil(rows_g / BM) * nt tiles, M-tiles fastest.
template <class T>
__global__ __launch_bounds__(256, 2) void gemm_grouped_kernel(const uint8_t* __restrict__ a,
                                                              const float* __restrict__ as,
                                                              const uint8_t* __restrict__ b,
                                                              const float* __restrict__ bs,
                                                              uint16_t* __restrict__ c,
                                                              const int32_t* __restrict__ off,
                                                              int G, int64_t N, int64_t K,
                                                              int nt) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * T::STAGE];
    const int64_t KB = K / kBlock;
    const int64_t NB = (N + kBlock - 1) / kBlock;
    int64_t total = 0;
    for (int g = 0; g < G; ++g) {
        const int64_t rows = (int64_t)off[g + 1] - off[g];
        total += ((rows + T::BM - 1) / T::BM) * nt;
    }
    for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
        int64_t start = 0;
        int g = 0;
        int64_t mtiles = 0;
        for (; g < G; ++g) {
            const int64_t rows = (int64_t)off[g + 1] - off[g];
            mtiles = (rows + T::BM - 1) / T::BM;
            if (t < start + mtiles * nt) break;
            start += mtiles * nt;
        }
        const int64_t local = t - start;
        const int64_t tm = local % mtiles;
        const int64_t tn = local / mtiles;
        gemm_tile<T>(a, as, b + (int64_t)g * N * K, bs + (int64_t)g * NB * KB, c,
                     (int64_t)off[g] + tm * T::BM, (int64_t)off[g + 1], tn * T::BN, N, K, lds);
    }
}

// ---------------------------------------------------------------------------
// Large-tile kernel: direct global -> LDS loads, 8 waves.
//
// WG tile BM x BN with WAVES_M x WAVES_N waves (wave tile WM x WN).  The A and
// B tiles of one 128-wide K block are fetched with global_load_lds_dwordx4:
// one wave instruction fills 1 KB of LDS (eight 128-byte rows), lane l writing
// bytes [16 l, 16 l + 16).  The XOR swizzle is applied on the source side:
// lane l of an instruction covering rows r0..r0+7 fetches logical chunk
// (l & 7) ^ ((l >> 3) & 7) of row r0 + (l >> 3), so LDS chunk c of row r holds
// logical chunk c ^ (r & 7), exactly the layout the fragment reads expect.
// The row scales of the K block arrive the same way (4 bytes per lane).
// Loads for K block kb+1 are issued before the MFMAs of block kb; one
// s_waitcnt + barrier per K block closes the step.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_>
struct BigTile {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NSTAGE = NSTAGE_;                  // LDS stages (prefetch distance NSTAGE-1)
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int A_BYTES = BM * kBlock, B_BYTES = BN * kBlock;
    // Row scales of one K block, permuted for the fragment layout: row 16 i + t
    // sits at float t * SPITCH + i.  SPITCH = BM/16 + 4 keeps the 16 lanes of a
    // read on distinct bank groups and each lane's TM values 16-byte aligned.
    static constexpr int SPITCH = BM / 16 + 4;
    static constexpr int S_FLOATS = 16 * SPITCH;
    static constexpr int S_INSTR = (S_FLOATS + 63) / 64;   // 256-byte scale instructions
    // every wave issues one scale instruction (waves past S_INSTR fill unused
    // slots), so all waves have the same number of loads in flight per stage
    static constexpr int S_BYTES = (WAVES * 256 + 1023) / 1024 * 1024;
    static constexpr int LOADS_PER_STAGE = BM / 8 / WAVES + BN / 8 / WAVES + 1;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static constexpr int A_INSTR = BM / 8 / WAVES;          // 1 KB instructions per wave for A
    static constexpr int B_INSTR = BN / 8 / WAVES;
    static_assert(BM % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "tile rows must split over waves");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one scale block");
    static_assert(S_INSTR <= WAVES, "one scale instruction per wave at most");
    static_assert(TM % 4 == 0, "scales are read four at a time");
    static_assert(STAGE % 1024 == 0, "stages stay 1 KB aligned");
    static_assert(NSTAGE >= 2 && NSTAGE * STAGE <= 160 * 1024, "stages must fit in LDS");
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

__device__ __forceinline__ void load_lds16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds((gbl_void_t)src, (lds_void_t)lds_dst, 4, 0, 0);
}

// The MFMA is issued with the weight fragment as its first operand and the
// activation fragment as its second, so the 16 x 16 result is C^T: lane l
// holds output row m = l & 15 of the sub-tile and the four consecutive columns
// n = 4 (l >> 4) + 0..3.  Each lane therefore needs one activation scale per
// sub-tile row block, and the epilogue writes 8 contiguous bytes per sub-tile.
template <class T>
__device__ __forceinline__ void gemm_tile_big(const uint8_t* __restrict__ a,
                                              const float* __restrict__ as,
                                              const uint8_t* __restrict__ b,
                                              const float* __restrict__ bs,
                                              uint16_t* __restrict__ c, int64_t m0, int64_t m_end,
                                              int64_t n0, int64_t N, int64_t K, uint8_t* lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / T::WAVES_N) * T::WM;
    const int wn0 = (wave % T::WAVES_N) * T::WN;
    const int64_t KB = K / kBlock;
    const int64_t NB = (N + kBlock - 1) / kBlock;

    // Direct-load sources.  Instruction i of this wave fills LDS rows
    // r0 .. r0+7 (r0 = 8 * (wave * INSTR + i)); lane l writes physical chunk
    // l & 7 of row r0 + (l >> 3), which must hold logical chunk
    // (l & 7) ^ swz(row).  Offsets are 32-bit, relative to the tile's
    // first row, so the K-block step is one scalar add on the base pointer.
    const int lrow = lane >> 3;
    uint32_t a_off[T::A_INSTR], b_off[T::B_INSTR];
#pragma unroll
    for (int i = 0; i < T::A_INSTR; ++i) {
        const int row = (wave * T::A_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        int64_t grow = m0 + row;
        grow = grow < m_end ? grow : m_end - 1;
        a_off[i] = (uint32_t)((grow - m0) * K) + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < T::B_INSTR; ++i) {
        const int row = (wave * T::B_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        int64_t gcol = n0 + row;
        gcol = gcol < N ? gcol : N - 1;
        b_off[i] = (uint32_t)((gcol - n0) * K) + chunk * 16;
    }
    // scale slot p = t * SPITCH + i holds row 16 i + t (pad slots load row 0)
    uint32_t s_off = 0;
    {
        const int p = wave * 64 + lane;
        const int t = p / T::SPITCH, i = p % T::SPITCH;
        int row = (t < 16 && i < T::BM / 16) ? 16 * i + t : 0;
        int64_t grow = m0 + row;
        grow = grow < m_end ? grow : m_end - 1;
        s_off = (uint32_t)((grow - m0) * KB);
    }
    const uint8_t* a_tile = a + m0 * K;
    const uint8_t* b_tile = b + n0 * K;
    const float* s_tile = as + m0 * KB;
    int64_t nblk = (n0 + wn0) >> 7;
    nblk = nblk < NB ? nblk : NB - 1;
    const float* sb_src = bs + nblk * KB;

    auto issue = [&](int64_t kb, int stage) {
        uint8_t* base = lds + stage * T::STAGE;
        const uint8_t* ak = a_tile + kb * kBlock;
        const uint8_t* bk = b_tile + kb * kBlock;
#pragma unroll
        for (int i = 0; i < T::A_INSTR; ++i)
            load_lds16(ak + a_off[i], base + (wave * T::A_INSTR + i) * 1024);
#pragma unroll
        for (int i = 0; i < T::B_INSTR; ++i)
            load_lds16(bk + b_off[i], base + T::A_BYTES + (wave * T::B_INSTR + i) * 1024);
        load_lds4(s_tile + kb + s_off, base + T::A_BYTES + T::B_BYTES + wave * 256);
    };

    v4f acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // prologue: K blocks 0 .. NSTAGE-2 in flight
#pragma unroll
    for (int st = 0; st + 1 < T::NSTAGE; ++st)
        if (st < KB) issue(st, st);

    const int lr = lane & 15;
    const int lk = (lane >> 4) * 2;
    const int off0 = ((lk ^ swz(lr)) << 4);
    const int off1 = (((lk + 1) ^ swz(lr)) << 4);
    const int sread = lr * T::SPITCH + wm0 / 16;

    int cur = 0;
    for (int64_t kb = 0; kb < KB; ++kb) {
        // this wave's loads of block kb are done once at most the later
        // blocks' loads are outstanding; the barrier then makes every wave's
        // loads visible and guarantees stage (kb-1) is no longer being read
        if (kb + T::NSTAGE - 2 < KB)
            wait_vmcnt<T::LOADS_PER_STAGE * (T::NSTAGE - 2)>();
        else
            wait_vmcnt<0>();
        barrier_lds();
        if (kb + T::NSTAGE - 1 < KB) {
            int st = cur + T::NSTAGE - 1;
            st = st >= T::NSTAGE ? st - T::NSTAGE : st;
            issue(kb + T::NSTAGE - 1, st);
        }

        const uint8_t* As = lds + cur * T::STAGE;
        const uint8_t* Bs = As + T::A_BYTES;
        const float* Ss = (const float*)(Bs + T::B_BYTES);
        v8i fb[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const uint8_t* r = Bs + (wn0 + 16 * j + lr) * kBlock;
            fb[j] = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
        }
        const float sbv = sb_src[kb];
        float sc[T::TM];
#pragma unroll
        for (int i = 0; i < T::TM; i += 4) {
            const v4f s4 = *(const v4f*)(Ss + sread + i);
            sc[i] = s4[0] * sbv; sc[i + 1] = s4[1] * sbv; sc[i + 2] = s4[2] * sbv; sc[i + 3] = s4[3] * sbv;
        }
        // MFMAs of sub-tile row i are issued before the fold of row i - 1, so
        // each block product has TN MFMAs of distance before it is read; the
        // A fragment of row i + 1 is read from LDS while row i multiplies.
        v4f prev[T::TN];
        v8i fa_next;
        {
            const uint8_t* r = As + (wm0 + lr) * kBlock;
            fa_next = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const v8i fa = fa_next;
            if (i + 1 < T::TM) {
                const uint8_t* r = As + (wm0 + 16 * (i + 1) + lr) * kBlock;
                fa_next = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
            }
            v4f cur[T::TN];
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[j], fa, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if (i > 0) {
#pragma unroll
                for (int j = 0; j < T::TN; ++j) acc[i - 1][j] = prev[j] * sc[i - 1] + acc[i - 1][j];
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j) prev[j] = cur[j];
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[T::TM - 1][j] = prev[j] * sc[T::TM - 1] + acc[T::TM - 1][j];
        // Instruction order of this K block, given to the scheduler: the
        // direct loads, the B / scale / first-A reads and the scale products,
        // then per sub-tile row the next A read and TN x (1 MFMA, 4 fold FMAs).
        __builtin_amdgcn_sched_group_barrier(0x020, T::A_INSTR + T::B_INSTR + 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::TN + T::TM / 4 + 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, T::TM, 0);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            if (i + 1 < T::TM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 4 * T::TN, 0);
        cur = cur + 1 == T::NSTAGE ? 0 : cur + 1;
    }

    // epilogue: lane holds row m0 + wm0 + 16 i + lr, columns n0 + wn0 + 16 j + 4 (lane >> 4) + 0..3
    const int cq = 4 * (lane >> 4);
    const bool interior = (m0 + T::BM <= m_end) && (n0 + T::BN <= N);
    const bool vec = interior && (N % 4 == 0) && (((uintptr_t)c & 7u) == 0);
    if (vec) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            uint16_t* crow = c + (m0 + wm0 + 16 * i + lr) * N + n0 + wn0 + cq;
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
                    const int64_t col = n0 + wn0 + 16 * j + cq + r;
                    if (row < m_end && col < N)
                        c[row * N + col] = (uint16_t)bf16_rne_bits(acc[i][j][r]);
                }
            }
        }
    }
}

// Maps a workgroup id to a tile so that the workgroups resident on one XCD
// (ids are dealt round-robin over the 8 XCDs) work on a compact block of
// tiles: ids are first regrouped XCD by XCD, then walked in bands of GM
// M-tiles (M fastest inside a band).
__device__ __forceinline__ void tile_of(int id, int nwg, int mt, int nt, int& tm, int& tn) {
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
__global__ __launch_bounds__(T::THREADS, 1) void gemm_big_kernel(const uint8_t* __restrict__ a,
                                                                 const float* __restrict__ as,
                                                                 const uint8_t* __restrict__ b,
                                                                 const float* __restrict__ bs,
                                                                 uint16_t* __restrict__ c,
                                                                 int64_t M, int64_t N, int64_t K,
                                                                 int mt, int nt) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T::NSTAGE * T::STAGE];
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, mt, nt, tm, tn);
    gemm_tile_big<T>(a, as, b, bs, c, (int64_t)tm * T::BM, M, (int64_t)tn * T::BN, N, K, lds);
}

using TileLarge = Tile<128, 128>;
using TileSmall = Tile<64, 64>;

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

using BigSquare = BigTile<256, 256, 2, 4, 2>;   // 8 waves of 128 x 64, 2 stages
using BigWide = BigTile<256, 128, 4, 2, 3>;     // 8 waves of 64 x 64, 3 stages

template <class T>
static void launch_big(const void* a, const float* as, const void* b, const float* bs, void* c,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
    hipLaunchKernelGGL(gemm_big_kernel<T>, dim3(mt * nt), dim3(T::THREADS), 0, stream,
                       (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, nt);
}

// Which kernel configuration serves an M x N x K problem (the tile table).
GemmConfig gemm_config(int64_t M, int64_t N, int64_t /*K*/) {
    const int64_t cus = device_cu_count();
    const int64_t tiles_sq = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t tiles_wide = ((M + 255) / 256) * ((N + 127) / 128);
    if (M > 128 && tiles_sq >= 2 * cus) return GemmConfig::kBig256x256;
    if (M > 128 && tiles_wide >= cus / 2) return GemmConfig::kBig256x128;
    if (M <= 64) return GemmConfig::kReg64x64;
    return GemmConfig::kReg128x128;
}

const char* gemm_config_name(GemmConfig cfg) {
    switch (cfg) {
        case GemmConfig::kBig256x256: return "lds-direct 256x256, 8 waves of 128x64";
        case GemmConfig::kBig256x128: return "lds-direct 256x128, 8 waves of 64x64";
        case GemmConfig::kReg64x64: return "register-staged 64x64, 4 waves of 32x32";
        case GemmConfig::kReg128x128: return "register-staged 128x128, 4 waves of 64x64";
    }
    return "unknown";
}

hipError_t launch_gemm(const void* a, const float* as, const void* b, const float* bs, void* c,
                       int64_t M, int64_t N, int64_t K, void* /*workspace*/,
                       size_t /*workspace_bytes*/, hipStream_t stream) {
    switch (gemm_config(M, N, K)) {
        case GemmConfig::kBig256x256:
            launch_big<BigSquare>(a, as, b, bs, c, M, N, K, stream);
            break;
        case GemmConfig::kBig256x128:
            launch_big<BigWide>(a, as, b, bs, c, M, N, K, stream);
            break;
        case GemmConfig::kReg64x64: {
            using T = TileSmall;
            const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
            hipLaunchKernelGGL(gemm_kernel<T>, dim3(mt * nt), dim3(256), 0, stream,
                               (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K,
                               mt, nt);
            break;
        }
        case GemmConfig::kReg128x128: {
            using T = TileLarge;
            const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
            hipLaunchKernelGGL(gemm_kernel<T>, dim3(mt * nt), dim3(256), 0, stream,
                               (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K,
                               mt, nt);
            break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_gemm_grouped(const void* a, const float* as, const void* b, const float* bs,
                               void* c, const int32_t* off, int32_t G, int64_t total_M,
                               int64_t N, int64_t K, hipStream_t stream) {
    using T = TileLarge;
    const int nt = (int)((N + T::BN - 1) / T::BN);
    const int64_t max_tiles = ((total_M + T::BM - 1) / T::BM + G) * (int64_t)nt;
    const int64_t cap = (int64_t)device_cu_count() * 2;
    const int grid = (int)(max_tiles < cap ? max_tiles : cap);
    hipLaunchKernelGGL(gemm_grouped_kernel<T>, dim3(grid), dim3(256), 0, stream,
                       (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, off, (int)G, N,
                       K, nt);
    return hipGetLastError();
}

}  // namespace bfp8
