// grouped.hip - the grouped block-scaled fp8 GEMM (one GPU's share of routed
// experts) on gfx950: rows [off[g], off[g+1]) of a times expert g's weight,
// c[m, n] = bf16( sum_kb P_kb[m, n] * a_s[m, kb] * b_s[g][n/128, kb] ), with the
// group offsets read on the device.
#include "device_codec.hpp"
#include "internal.hpp"
#include "tile_common.hpp"

namespace bfp8 {

// ------------------------------------------------------------- grouped GEMM
//
// One persistent launch over every group's tiles ("Behavior traces", MoE
// trace; pyshine tour, "Honest Limits": one fused grouped GEMM instead of a
// loop over experts).  Routed experts hold about as many rows as one 256-row
// tile, a few more or fewer, and the weights are streamed from HBM once per
// M-tile.  So a tile here is 256 rows plus up to 64 more: the group's last
// tile takes a remainder of at most 64 rows into the same K loop (the same B
// blocks in LDS), and every group's weight is read once.  A group of n rows
// gets n / 256 tiles when n % 256 <= 64 (the last one tall), else one more,
// partial, tile.
//
// Tile: 320 x 256 at most, 8 waves in 2 (M) x 4 (N).  Wave (wm, wn) owns
// columns 64 wn .. 64 wn + 63 and up to ten 16-row sub-tile rows: the main
// rows 128 wm + 16 i (i < 8) and the extra rows 256 + 16 wm + 32 x (x = 0, 1),
// so the two wave rows share a remainder.  A tile runs one of three variants
// (no extra row, one, or two per wave row), each a K loop without branches.
// LDS per stage: A (the ten sub-tile rows of wave row wm at rows 160 wm ..
// 160 wm + 159, so one base address and immediate offsets reach them all), B
// (256 rows), and one line of row scales and weight scales; every region is
// its own array, so the compiler sees that a fill of one stage never aliases
// the reads of the other.  Waves 0..3 issue the A and B loads of the next K
// block right after each block's barrier (waves 4..7 run one priority level
// up and only multiply).  Rows past the tile's valid rows, and weight rows
// past N, fall outside the buffer resources, which read them as zeros; they
// are never stored.  The weight is loaded with the non-temporal hint: each
// block is used once, and should not push the group's rows (shared by its
// N-tiles) out of L2.  The fold is acc += P * (a_s[row] * b_s) per 16 x 16
// block product, as in the dense tile, software-pipelined one MFMA deep.
struct GroupedTile {
    static constexpr int BM = 256, XM = 64, BN = 256;
    static constexpr int WAVES = 8, THREADS = 64 * WAVES, LOADERS = 4;
    static constexpr int WM = 128, WN = 64, TM = 8, TN = 4, TR_MAX = TM + XM / 32;
    static constexpr int WROWS = 16 * TR_MAX;                  // LDS rows per wave row (160)
    static constexpr int A_BYTES = 2 * WROWS * kBlock, B_BYTES = BN * kBlock;
    static constexpr int MAIN_INSTR = BM / 8 / LOADERS, B_INSTR = BN / 8 / LOADERS;
    // row scales: lane row t (0..15) of wave row wm, sub-tile row i sits at
    // float t * SP + 12 wm + i (16-byte aligned groups of four; SP / 4 odd, so
    // the 16 lanes of a read hit distinct bank groups); the 64-float weight-scale
    // line follows
    static constexpr int SP = 28, S_FLOATS = 16 * SP, S_INSTR = S_FLOATS / 64;
    static constexpr int SB_OFF = S_FLOATS, S_LINE = S_FLOATS + 64;
    static_assert(MAIN_INSTR % 2 == 0 && B_INSTR % 2 == 0, "instruction parity picks the offset");
    static_assert(S_FLOATS % 64 == 0 && S_INSTR < WAVES, "one scale instruction per wave");
    static_assert(2 * (A_BYTES + B_BYTES + 4 * S_LINE) <= 158 * 1024, "two stages fit in LDS");
};

struct GroupedLds {
    uint8_t* a[2];
    uint8_t* b[2];
    float* s[2];
};

// Tiles of a group of `rows` rows (see above).
__device__ __forceinline__ int64_t grouped_m_tiles(int64_t rows) {
    const int64_t full = rows / GroupedTile::BM, rem = rows - full * GroupedTile::BM;
    return full + ((rem > GroupedTile::XM || (rem > 0 && full == 0)) ? 1 : 0);
}

// Rows of group g: the device offsets clamped into [0, total_M] (and the end
// to at least the start), so offsets produced on the device can never send a
// tile outside the caller's buffers.
__device__ __forceinline__ void group_rows(const int32_t* __restrict__ off, int g,
                                           int64_t total_M, int64_t& lo, int64_t& hi) {
    int64_t a = off[g], b = off[g + 1];
    a = a < 0 ? 0 : (a > total_M ? total_M : a);
    b = b < a ? a : (b > total_M ? total_M : b);
    lo = a;
    hi = b;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Where tile t lies (tiles ordered group by group, N-tile by N-tile, M-tile
// fastest): the groups are scanned 64 at a time, one group per lane (a
// coalesced load of its offsets, its tile count, a wave prefix sum of the
// counts), so finding a tile costs one memory round trip per 64 groups.
// Every wave of the workgroup does the same scan; the results are
// wave-uniform.  Returns false when t lies past the last tile.
struct TileAt {
    int g;
    int64_t m0, m_end, n0;
};

__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ off, int G, int64_t total_M,
                                            int nt, int64_t t, TileAt& at) {
    // the lane id is hidden from the compiler here, so nothing of this scan is hoisted
    // out of the caller's tile loop to stay live (in VGPRs) through every tile's K loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    int64_t base = 0;
    for (int g0 = 0; g0 < G; g0 += 64) {
        const int g = g0 + lane;
        int64_t lo = 0, hi = 0;
        int mcount = 0;
        if (g < G) {
            group_rows(off, g, total_M, lo, hi);
            mcount = (int)grouped_m_tiles(hi - lo);
        }
        // tile counts of 64 groups: below 2^31 (rows < 2^31 per call, N-tiles < 2^16)
        const int cnt = mcount * nt;
        int inc = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(inc, d);
            if (lane >= d) inc += v;
        }
        const int64_t start = base + (inc - cnt);
        const unsigned long long hit = __ballot(g < G && t >= start && t < start + cnt);
        if (hit != 0ull) {
            const int src = __builtin_amdgcn_readfirstlane(__ffsll(hit) - 1);
            const int64_t rest = t - uniform64(__shfl(start, src));
            const int64_t mc = __builtin_amdgcn_readfirstlane(__shfl(mcount, src));
            const int64_t glo = uniform64(__shfl(lo, src)), ghi = uniform64(__shfl(hi, src));
            const int64_t tm = rest % mc;
            at.g = g0 + src;
            at.m0 = glo + tm * GroupedTile::BM;
            at.m_end = (tm == mc - 1) ? ghi : at.m0 + GroupedTile::BM;   // the last tile takes the rest
            at.n0 = (rest / mc) * GroupedTile::BN;
            return true;
        }
        base += __builtin_amdgcn_readfirstlane(__shfl(inc, 63));
    }
    return false;
}

// Row of the tile that sub-tile row i of wave row wm starts at.
__device__ __forceinline__ int grouped_row(int wm, int i) {
    return i < GroupedTile::TM ? GroupedTile::WM * wm + 16 * i : GroupedTile::BM + 16 * wm + 32 * (i - GroupedTile::TM);
}

// One tile with TX extra sub-tile rows in this wave's row (wave row 0 takes
// its first extra row past 256 rows, wave row 1 past 272, the second ones past
// 288 and 304); the loading waves, in wave row 0, load the A rows of their TX.
// Each variant runs its K loop with no branch inside (a branch would make the
// compiler wait for the next block's loads before the LDS reads that follow
// it); rows past the tile's valid rows are multiplied (their inputs read as
// zeros) but never stored.
template <int TX>
__device__ __forceinline__ void grouped_tile(const uint8_t* __restrict__ a,
                                             const float* __restrict__ as,
                                             const uint8_t* __restrict__ b,
                                             const float* __restrict__ bs,
                                             uint16_t* __restrict__ c, int64_t m0, int64_t m_end,
                                             int64_t n0, int64_t N, int64_t K, const GroupedLds& L) {
    using T = GroupedTile;
    constexpr int TR = T::TM + TX;                         // sub-tile rows per wave
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4;
    const int64_t KB = K / kBlock;
    const int64_t NBK = (N + kBlock - 1) / kBlock;
    const int rows_a = (int)(m_end - m0);                 // 1 .. 256 + 32 TX
    const int rows_b = (int)((N - n0) < T::BN ? (N - n0) : T::BN);
    // rows past rows_a / rows_b lie outside these resources and read as zeros
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a + m0 * K, (uint64_t)rows_a * K);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(b + n0 * K, (uint64_t)rows_b * K);
    const __amdgpu_buffer_rsrc_t rs_as = make_rsrc(as + m0 * KB, (uint64_t)rows_a * KB * 4);
    const __amdgpu_buffer_rsrc_t rs_bs = make_rsrc(bs, (uint64_t)NBK * KB * 4);

    // Loads of loading wave w < LOADERS.  Main A instruction i (k = 8 w + i) brings tile rows
    // 8 k .. 8 k + 7 (LDS rows 160 (k / 16) + 8 (k % 16) ..); extra A instruction x (e = w +
    // 4 x < 4 TX) tile rows 256 + 8 e .. (LDS rows 160 ((e / 2) % 2) + 128 + 16 (e / 4) +
    // 8 (e % 2) ..); B instruction i (k = 8 w + i) weight rows 8 k ... Lane l writes
    // physical chunk l & 7 of the LDS row + (l >> 3), which holds logical chunk
    // (l & 7) ^ swz(LDS row); with eight rows per instruction swz = (l >> 3) ^ (parity of
    // k, or of e).  The per-lane offsets depend only on that parity; the eight-row steps go
    // into the scalar offset.
    const int lrow = lane >> 3;
    uint32_t voff_a[2], voff_b[2], voff_x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        voff_a[p] = (uint32_t)((wave * T::MAIN_INSTR * 8 + lrow) * K + (((lane & 7) ^ lrow ^ p) * 16));
        voff_b[p] = (uint32_t)((wave * T::B_INSTR * 8 + lrow) * K + (((lane & 7) ^ lrow ^ p) * 16));
    }
    voff_x = (uint32_t)((T::BM + 8 * wave + lrow) * K + (((lane & 7) ^ lrow ^ (wave & 1)) * 16));
    // row-scale slot q = wave * 64 + lane (waves < S_INSTR): lane row t = q / SP, wave row
    // and sub-tile row from q % SP; unused slots load row 0
    uint32_t as_off;
    {
        const int q = wave * 64 + lane, t = q / T::SP, k = q % T::SP;
        const int r_wm = k / 12, r_i = k % 12;
        const int row = (r_wm < 2 && r_i < T::TR_MAX) ? grouped_row(r_wm, r_i) + t : 0;
        as_off = (uint32_t)(row * KB * 4);
    }
    uint32_t bs_off;
    {
        int64_t nb = (n0 >> 7) + lane;
        nb = nb < NBK ? nb : NBK - 1;
        bs_off = (uint32_t)(nb * KB * 4);
    }

    const uint32_t k8 = (uint32_t)(8 * K);                 // byte step of eight rows
    auto issue = [&](int64_t kb, auto S_) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        const uint32_t ko = (uint32_t)(kb * kBlock);
        uint8_t* la = L.a[S];
        uint8_t* lb = L.b[S];
        if (wave < T::LOADERS) {
            // the scalar offset advances by eight rows per instruction; the empty asm keeps
            // the compiler from precomputing every instruction's offset into its own SGPR
            uint32_t so = ko;
#pragma unroll
            for (int i = 0; i < T::MAIN_INSTR; ++i) {
                const int k = wave * T::MAIN_INSTR + i;
                buf_lds16(rs_a, voff_a[i & 1], so, la + ((k >> 4) * T::WROWS + (k & 15) * 8) * kBlock);
                so += k8;
                asm volatile("" : "+s"(so));
            }
#pragma unroll
            for (int x = 0; x < TX; ++x) {
                const int e = wave + 4 * x;
                buf_lds16(rs_a, voff_x, ko + (uint32_t)(x * 4) * k8,
                          la + (((e >> 1) & 1) * T::WROWS + T::TM * 16 + 16 * (e >> 2) + 8 * (e & 1)) * kBlock);
            }
            so = ko;
#pragma unroll
            for (int i = 0; i < T::B_INSTR; ++i) {
                buf_lds16_nt(rs_b, voff_b[i & 1], so, lb + (wave * T::B_INSTR + i) * 1024);
                so += k8;
                asm volatile("" : "+s"(so));
            }
        }
        const uint32_t so = (uint32_t)(kb * 4);
        if (wave < T::S_INSTR) buf_lds4(rs_as, as_off, so, L.s[S] + wave * 64);
        if (wave == T::WAVES - 1) buf_lds4(rs_bs, bs_off, so, L.s[S] + T::SB_OFF);
    };

    v4f acc[TR][T::TN];
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // a workgroup walking several tiles must not refill a stage a slower wave still reads
    wait_vmcnt<0>();
    barrier_lds();
    issue(0, StageId<0>{});

    const int lr = lane & 15;
    const int lk = (lane >> 4) * 2;
    const int off0 = ((lk ^ swz(lr)) << 4);
    const int off1 = (((lk + 1) ^ swz(lr)) << 4);
    const int arow = (wm * T::WROWS + lr) * kBlock;        // this lane's row of sub-tile row 0
    const int brow = (T::WN * wn + lr) * kBlock;
    const int sread = lr * T::SP + 12 * wm;

    auto step = [&](int64_t kb, auto S_) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        wait_vmcnt<0>();              // this wave's loads of block kb
        barrier_lds();                // everyone's loads of kb landed; block kb - 1 fully read
        if (kb + 1 < KB) issue(kb + 1, StageId<1 - S>{});
        const uint8_t* As = L.a[S] + arow;
        const uint8_t* Bs = L.b[S] + brow;
        const float* Ss = L.s[S];
        // The block as one software pipeline over the (row, column) sub-tiles: each MFMA is
        // followed by the four folds of the previous sub-tile's product, which has landed
        // while this MFMA was issued, so neither the MFMA pipe nor the wave waits on a fold;
        // two product registers alternate.  The next row's A fragment is read after the
        // row's first MFMA, the B fragments during row 0's MFMAs.
        v8i fb[T::TN];
        v8i fa, fa_nxt;
        fa_nxt = frag_from(*(const uint4*)(As + off0), *(const uint4*)(As + off1));
        fb[0] = frag_from(*(const uint4*)(Bs + off0), *(const uint4*)(Bs + off1));
        const v4f s0 = *(const v4f*)(Ss + sread), s1 = *(const v4f*)(Ss + sread + 4);
        float2 s2 = float2{0.f, 0.f};
        if constexpr (TX > 0) s2 = *(const float2*)(Ss + sread + 8);
        const float sbv = Ss[T::SB_OFF + (wn >> 1)];
        __builtin_amdgcn_sched_barrier(0);
        v4f pr[2];
        float sc_prev = 0.f;
#pragma unroll
        for (int i = 0; i < TR; ++i) {
            fa = fa_nxt;
            const float sa = i < 4 ? s0[i] : (i < 8 ? s1[i - 4] : (i == 8 ? s2.x : s2.y));
            const float sc = sa * sbv;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int idx = i * T::TN + j;
                pr[idx & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[j], fa, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                if (i == 0 && j + 1 < T::TN) {
                    const uint8_t* q = Bs + 16 * (j + 1) * kBlock;
                    fb[j + 1] = frag_from(*(const uint4*)(q + off0), *(const uint4*)(q + off1));
                }
                if (j == 0 && i + 1 < TR) {
                    const uint8_t* r = As + 16 * (i + 1) * kBlock;
                    fa_nxt = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
                }
                if (idx > 0) {
                    const int pi = (idx - 1) / T::TN, pj = (idx - 1) % T::TN;
                    acc[pi][pj] = pr[(idx - 1) & 1] * (pj == T::TN - 1 ? sc_prev : sc) + acc[pi][pj];
                }
                // pin the order: this MFMA, the reads, the previous product's folds
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if ((i == 0 && j + 1 < T::TN) || (j == 0 && i + 1 < TR))
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                if (idx > 0 && j == 0) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
                if (idx > 0 && j > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            sc_prev = sc;
        }
        acc[TR - 1][T::TN - 1] = pr[(TR * T::TN - 1) & 1] * sc_prev + acc[TR - 1][T::TN - 1];
        __builtin_amdgcn_sched_barrier(0);
    };

    if (wave >= 4) __builtin_amdgcn_s_setprio(1);
    for (int64_t kb = 0; kb < KB; kb += 2) {
        step(kb, StageId<0>{});
        if (kb + 1 < KB) step(kb + 1, StageId<1>{});
    }
    if (wave >= 4) __builtin_amdgcn_s_setprio(0);

    // epilogue: lane holds row m0 + grouped_row(wm, i) + lr, columns n0 + 64 wn + 16 j + 4 (lane >> 4) + 0..3
    const int cq = 4 * (lane >> 4);
    const bool fast = (N % 4 == 0) && (((uintptr_t)c & 7u) == 0) && (n0 + T::BN <= N);
    uint16_t* cbase = c + m0 * N + n0 + T::WN * wn + cq;
#pragma unroll
    for (int i = 0; i < TR; ++i) {
        const int r = grouped_row(wm, i) + lr;
        if (r >= rows_a) continue;
        uint16_t* crow = cbase + (int64_t)r * N;
        if (fast) {
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                uint2 v;
                v.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                v.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                *(uint2*)(crow + 16 * j) = v;
            }
        } else {
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + T::WN * wn + 16 * j + cq + e < N)
                        crow[16 * j + e] = (uint16_t)bf16_rne_bits(acc[i][j][e]);
        }
    }
}

// Persistent: workgroups are dealt round-robin over the 8 XCDs, and in each
// round the workgroups of one XCD take a contiguous run of tiles, so one XCD
// works on a few groups' rows (shared by their N-tiles through L2) at a time.
__global__ __launch_bounds__(GroupedTile::THREADS, 1) void gemm_grouped_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, uint16_t* __restrict__ c, const int32_t* __restrict__ off,
    int G, int64_t total_M, int64_t N, int64_t K, int nt) {
    using T = GroupedTile;
    __shared__ __attribute__((aligned(1024))) uint8_t la0[T::A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t la1[T::A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lb0[T::B_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lb1[T::B_BYTES];
    __shared__ __attribute__((aligned(256))) float ls0[T::S_LINE];
    __shared__ __attribute__((aligned(256))) float ls1[T::S_LINE];
    const GroupedLds L = {{la0, la1}, {lb0, lb1}, {ls0, ls1}};
    const int64_t KB = K / kBlock;
    const int64_t NB = (N + kBlock - 1) / kBlock;
    const int nwg = gridDim.x;                    // a multiple of 8
    const int xcd = blockIdx.x % 8, local = blockIdx.x / 8;
    const int per_xcd = nwg / 8;
    for (int64_t round = 0;; ++round) {
        const int64_t t = round * nwg + (int64_t)xcd * per_xcd + local;
        TileAt at;
        if (!locate_tile(off, G, total_M, nt, t, at)) break;           // past the last tile
        const uint8_t* bg = b + (int64_t)at.g * N * K;
        const float* bsg = bs + (int64_t)at.g * NB * KB;
        // extra sub-tile rows this wave row needs (its rows 256 + 16 wm + 32 x hold tile rows);
        // the loading waves are in wave row 0, which needs at least as many as wave row 1,
        // so they load every extra row the tile has
        const int64_t rows = at.m_end - at.m0;
        const int wm = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6) / 4);
        const int tx = (rows > T::BM + 16 * wm ? 1 : 0) + (rows > T::BM + 32 + 16 * wm ? 1 : 0);
        if (tx == 0)
            grouped_tile<0>(a, as, bg, bsg, c, at.m0, at.m_end, at.n0, N, K, L);
        else if (tx == 1)
            grouped_tile<1>(a, as, bg, bsg, c, at.m0, at.m_end, at.n0, N, K, L);
        else
            grouped_tile<2>(a, as, bg, bsg, c, at.m0, at.m_end, at.n0, N, K, L);
    }
}

hipError_t launch_gemm_grouped(const void* a, const float* as, const void* b, const float* bs,
                               void* c, const int32_t* off, int32_t G, int64_t total_M,
                               int64_t N, int64_t K, hipStream_t stream) {
    using T = GroupedTile;
    const int nt = (int)((N + T::BN - 1) / T::BN);
    // an upper bound of the tile count (the exact one depends on the device offsets):
    // at most total_M / 256 full tiles plus one more per group
    const int64_t max_tiles = (total_M / T::BM + G) * (int64_t)nt;
    const int64_t cus = device_cu_count();
    int64_t grid = max_tiles < cus ? max_tiles : cus;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL(gemm_grouped_kernel, dim3((unsigned)grid), dim3(T::THREADS), 0, stream,
                       (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, off, (int)G,
                       total_M, N, K, nt);
    return hipGetLastError();
}

}  // namespace bfp8
