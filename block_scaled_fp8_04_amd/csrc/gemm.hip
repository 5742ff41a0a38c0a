// gemm.hip - block-scaled fp8 GEMM on gfx950 (the grouped GEMM is in grouped.hip).
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
//  * Large tiles (BigTile): 256x256 (8 waves of 128x64, 2 LDS stages),
//    256x128 (8 waves of 64x64, 3 stages) and 128x128 (4 waves of 64x64,
//    2 stages, built for two workgroups per CU).  A and B rows of one K block
//    go straight from global memory into LDS with buffer loads; the stages are
//    distinct LDS arrays and the K loop is unrolled by the stage count, so
//    every stage is named at compile time.  A vmcnt-counted wait and one
//    barrier open each K block.
//  * Wave roles in the eight-wave tiles: waves w and w + 4 share a SIMD, and
//    waves 4..7 run one priority level up.  In the two-stage 256x256 tile
//    waves 0..3 also issue all of the tile's A and B loads, so waves 4..7
//    only multiply.
//  * Large problems with a workspace whose last round of 256x256 tiles would
//    run at most half full split those tiles over K into the workspace
//    (gemm_tail_kernel) and add the halves in order (tail_reduce_kernel).
//  * LDS rows are 128 bytes; the eight 16-byte chunks of row r are stored at
//    chunk position (chunk ^ swz(r)) (see swz below), so the 16 rows read
//    together by a fragment load (same logical chunk) hit no bank twice.
//  * MFMA operand layout: lane l supplies row (l & 15) of the sub-tile and the
//    32 K-bytes starting at 32 * (l >> 4), for A and B alike, so each K index
//    pairs the same position of A and B.  Operands go weight-first, so the
//    16x16 result is C^T: lane l holds output row (l & 15) and the four
//    consecutive columns 4 (l >> 4) + 0..3.
//  * Skinny problems (M <= 64, or M <= 256 with at most 32 tiles of 128 x 128)
//    with a workspace use split-K (gemm_skinny_kernel and a fixed-order
//    reduction).
//  * Rows past M and columns past N read a clamped, valid row; partial tiles
//    run the same K loop as full ones and only their stores are guarded.
#include <mutex>
#include <type_traits>

#include "device_codec.hpp"
#include "internal.hpp"
#include "tile_common.hpp"

namespace bfp8 {

// Adds the split-K partial sums ws[0..splits)[M][N] in index order (a fixed
// order, so results are reproducible) and rounds to bf16.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ ws,
                                                           uint16_t* __restrict__ c,
                                                           int64_t MN, int splits) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (MN % 4 == 0 && ((uintptr_t)c & 7u) == 0) {
        const int64_t n4 = MN / 4;
        for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
            // loads of up to 8 splits are issued together, then added in index order
            v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
            for (int sp0 = 0; sp0 < splits; sp0 += 8) {
                v4f part[8];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (sp0 + q < splits) part[q] = ((const v4f*)(ws + (int64_t)(sp0 + q) * MN))[i];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (sp0 + q < splits) sum = (sp0 + q == 0) ? part[q] : sum + part[q];
            }
            uint2 o;
            o.x = pack_bf16x2(sum[0], sum[1]);
            o.y = pack_bf16x2(sum[2], sum[3]);
            ((uint2*)c)[i] = o;
        }
        return;
    }
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += stride) {
        float sum = ws[i];
        for (int sp = 1; sp < splits; ++sp) sum += ws[(int64_t)sp * MN + i];
        c[i] = (uint16_t)bf16_rne_bits(sum);
    }
}

// Adds the tail's split partial sums ws[s][M][W] (W = N - n1) in split order
// and writes bf16 columns [n1, N) of c (row stride N).  W % 4 == 0.
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ ws,
                                                          uint16_t* __restrict__ c, int64_t M,
                                                          int64_t N, int64_t n1, int splits) {
    const int64_t W = N - n1, W4 = W / 4, total = M * W4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t row = i / W4, c4 = i - row * W4;
        v4f sum = ((const v4f*)ws)[i];
        for (int sp = 1; sp < splits; ++sp) sum = sum + ((const v4f*)(ws + (int64_t)sp * M * W))[i];
        uint2 o;
        o.x = pack_bf16x2(sum[0], sum[1]);
        o.y = pack_bf16x2(sum[2], sum[3]);
        *(uint2*)(c + row * N + n1 + 4 * c4) = o;
    }
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NSTAGE_>
struct BigTile {
    static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NSTAGE = NSTAGE_;                  // LDS stages (prefetch distance NSTAGE-1)
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    static constexpr int TM = WM / 16, TN = WN / 16;
    static constexpr int A_BYTES = BM * kBlock, B_BYTES = BN * kBlock;
    // Row scales of one K block, permuted for the fragment layout: row 16 i + t
    // sits at float t * SPITCH + i.  SPITCH is a multiple of 4 floats (each
    // lane's TM values 16-byte aligned) and an odd number of 16-byte units, so
    // the 16 lanes of a read fall on 16 distinct groups of 4 banks.
    static constexpr int SPITCH = ((BM / 16 + 4) / 4) % 2 == 1 ? BM / 16 + 4 : BM / 16 + 8;
    static constexpr int S_FLOATS = 16 * SPITCH;
    static constexpr int S_INSTR = (S_FLOATS + 63) / 64;   // 256-byte scale instructions
    // Wave w < S_INSTR loads the row-scale slots of its 256-byte part and
    // wave 0 the 256-byte weight-scale line (float t = the weight scale of
    // the tile's 128-column block t).  With three or more stages the waits
    // count loads per wave, so there every wave issues both instructions
    // (waves past S_INSTR fill slots nobody reads, every wave writes the same
    // weight scales) and all waves have the same loads in flight; with two
    // stages each wave waits for all of its own loads, and the fillers only
    // cost address-unit time (dropping them measured 4-6% faster).
    static constexpr int SB_OFF = WAVES * 256;
    static constexpr int S_BYTES = (WAVES * 256 + 256 + 1023) / 1024 * 1024;
    // Waves that issue the A and B row loads.  In the two-stage eight-wave
    // tiles waves 0..3 issue all of them and waves 4..7 (which run one
    // priority level up) only multiply: 3.5-4.6% faster on the dense shapes
    // than every wave loading its share (loads from waves 4..7, or waves 0..3
    // loading without the priority split, measured slower).  With more stages
    // every wave loads its share (the waits count loads per wave).
    static constexpr int LOADERS = (NSTAGE == 2 && WAVES == 8) ? 4 : WAVES;
    static constexpr int A_INSTR = BM / 8 / LOADERS;        // 1 KB instructions per loading wave for A
    static constexpr int B_INSTR = BN / 8 / LOADERS;
    static constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR + 2;

    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    // Workgroups per CU the kernels are built for: two for four-wave tiles whose stages fit
    // twice in LDS (registers then capped at 256 per lane), so that one workgroup's waves
    // keep the SIMDs busy while the other's wait at its barrier; else one.
    static constexpr int OCC = (WAVES == 4 && 2 * NSTAGE * STAGE <= 160 * 1024) ? 2 : 1;
    static_assert(BM % (8 * LOADERS) == 0 && BN % (8 * LOADERS) == 0,
                  "tile rows must split over the loading waves");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one scale block");
    static_assert(S_INSTR <= WAVES, "one scale instruction per wave at most");
    static_assert(TM % 4 == 0, "scales are read four at a time");
    static_assert(BN / 128 <= 64, "weight scales fit one 64-float line");
    static_assert(STAGE % 1024 == 0, "stages stay 1 KB aligned");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4 && NSTAGE * STAGE <= 158 * 1024, "stages must fit in LDS");
};

// The LDS stages of a large tile are distinct __shared__ arrays, and the K
// loop is unrolled by the stage count, so every read and every
// direct-to-LDS fill names its stage at compile time.  The compiler can then
// see that a fill of one stage never aliases the reads of another, and it
// waits on LDS reads only for the reads it needs (with one shared array it
// drains every outstanding LDS read before each use).
template <class T>
struct Stages {
    uint8_t* p[4];
    // The split schedule (below) keeps each stage's weight rows and scales in an
    // array of their own, b[s]; p[s] then holds only the A rows.  Null otherwise.
    uint8_t* b[4];
};
// The MFMA is issued with the weight fragment as its first operand and the
// activation fragment as its second, so the 16 x 16 result is C^T: lane l
// holds output row m = l & 15 of the sub-tile and the four consecutive columns
// n = 4 (l >> 4) + 0..3.  Each lane therefore needs one activation scale per
// sub-tile row block, and the epilogue writes 8 contiguous bytes per sub-tile.
// kGuard: some rows of this tile lie past m_end.  Their loads read the last
// valid row again, so the explicitly scheduled fold loop multiplies every row
// as in a full tile (finite values, never stored) and only the epilogue tests
// rows against m_end: a partial tile takes no longer than a full one.  The
// power-of-two-scale loop skips the MFMAs of each wave's 16-row sub-tile rows
// that lie entirely past m_end (a wave-uniform test).
// Where the tile's result goes (the epilogue mode): kEpiBf16 stores bf16 C;
// kEpiQuant writes act_quant of the bf16-rounded result, e4m3 codes q [M, N]
// and scales qs [M, N/128]; kEpiSwiglu multiplies a 64-row-interleaved
// [w1; w3] weight and writes act_quant of silu(w1 x) * (w3 x), q [M, N/2].
struct QuantOut {
    uint8_t* q;
    float* qs;
};
// kEpiF32: the tile multiplies K blocks [kb_lo, kb_hi) only and stores its
// fp32 partial sums, row r and column n at ws[r * ldw + n - n_base].
struct PartialOut {
    int64_t kb_lo = 0, kb_hi = -1;      // kb_hi < 0: all K blocks
    float* ws = nullptr;
    int64_t ldw = 0, n_base = 0;
};
constexpr int kEpiBf16 = 0, kEpiQuant = 1, kEpiSwiglu = 2, kEpiF32 = 3;

// act_quant fused into the GEMM epilogue ("Data flow", FP8 quantization
// bullet: the next linear() quantizes this output in 128-element blocks).
// Each result is first rounded to bf16 (the unfused path's stored output),
// so the codes and scales equal act_quant of the bf16 result bit for bit:
// the same block max, scale = max(amax, floor) / 448, correctly rounded
// quotient and e4m3 conversion.  A 128-column block of a row spans the 64
// columns of two neighbouring waves (wave and wave ^ 1): each wave reduces its
// part over its lanes, the two halves meet in LDS, and each wave writes its
// own 64 codes per row; the even wave writes the row's scale.  With a 16-byte
// aligned q the codes go through LDS first (each wave's WM rows of 64 bytes
// in the second stage, 16-byte chunks XOR-swizzled by row), so every store
// writes a whole 64-byte row piece, 16 bytes per lane; otherwise each lane
// stores its 4 bytes per sub-tile directly.  Requires N % 128 == 0, so
// blocks past N are whole and skipped.
template <class T>
__device__ __forceinline__ void quant_epilogue(v4f (&acc)[T::TM][T::TN], const QuantOut& qo,
                                               int64_t m0, int64_t m_end, int64_t n0, int64_t N,
                                               int wave, int wm0, int wn0, int lane,
                                               uint8_t* lds_scratch, uint8_t* cbuf) {
    static_assert(T::WN == 64, "a 128-column block spans two waves of 64 columns");
    static_assert(T::WAVES * T::WM * 64 <= T::STAGE, "the staged codes fit one stage");
    static_assert(T::WAVES / 2 * T::WM * 64 <= T::A_BYTES, "half the staged codes fit the A rows");
    const int lr = lane & 15, g = lane >> 4;
    float pm[T::TM];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[i][j][r] = bf16_round_f32(acc[i][j][r]);
                m = fmaxf(m, fabsf(acc[i][j][r]));
            }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        pm[i] = m;
    }
    // the stages are free once every wave has left the K loop
    float* part = (float*)lds_scratch;            // [WAVES][WM] partial row maxima
    __syncthreads();
    if (g == 0) {
#pragma unroll
        for (int i = 0; i < T::TM; ++i) part[wave * T::WM + 16 * i + lr] = pm[i];
    }
    __syncthreads();
    const bool block_valid = n0 + wn0 < N;          // N % 128 == 0: the whole block or none
    const int64_t nbq = N / kBlock;
    const bool staged = ((uintptr_t)qo.q & 15u) == 0;
#pragma unroll
    for (int i = 0; i < T::TM; ++i) {
        const float amax = fmaxf(pm[i], part[(wave ^ 1) * T::WM + 16 * i + lr]);
        const float s = fmaxf(amax, kAmaxFloor) / kE4m3Max;
        const float rcp = 1.0f / s;
        const int64_t row = m0 + wm0 + 16 * i + lr;
        if (row < m_end && block_valid) {
            const int r = 16 * i + lr;
            uint8_t* qrow = qo.q + row * N + n0 + wn0 + 4 * g;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const uint32_t codes = e4m3_encode4<true>(
                    quotient(acc[i][j][0], s, rcp), quotient(acc[i][j][1], s, rcp),
                    quotient(acc[i][j][2], s, rcp), quotient(acc[i][j][3], s, rcp));
                if (staged)
                    *(uint32_t*)(cbuf + r * 64 + ((j ^ ((r >> 2) & 3)) << 4) + 4 * g) = codes;
                else
                    *(uint32_t*)(qrow + 16 * j) = codes;
            }
            if (g == 0 && (wn0 & 127) == 0) qo.qs[row * nbq + ((n0 + wn0) >> 7)] = s;
        }
    }
    if (staged && block_valid) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int q = 0; q < T::WM / 16; ++q) {
            const int r = 16 * q + (lane >> 2), ch = lane & 3;
            const int64_t row = m0 + wm0 + r;
            if (row < m_end) {
                const uint4 v = *(const uint4*)(cbuf + r * 64 + ((ch ^ ((r >> 2) & 3)) << 4));
                *(uint4*)(qo.q + row * N + n0 + wn0 + ch * 16) = v;
            }
        }
    }
}

// The gated FFN's first GEMM with its activation and act_quant in the
// epilogue.  The weight is [w1; w3] interleaved by 64 rows (rows 128 t ..
// 128 t + 63 are w1 rows 64 t .., the next 64 are the matching w3 rows), so in
// a 256-column tile of the 2 x 4 wave layout, waves wn = 0, 2 hold w1 x (the
// gate g) and waves wn = 1, 3 hold w3 x (the up value u) for the same 128
// output columns, each lane at the same (row, column) as its partner's lane.
// Output: h = bf16( bf16( silu(g) ) * u ), the operations a bf16 model does
// on bf16 g and u (silu(x) = x / (1 + e^-x), evaluated in fp32 and rounded
// once); then act_quant of h's 128-column block exactly as quant_epilogue.
// The two waves of a pair (g and u of the same columns) split the rows: each
// hands the other, through LDS (lane-major, no bank conflicts), the values of
// the rows the other finishes, so silu and the quantization run on all eight
// waves (6% faster than the g waves alone on 4096 x 2048 x 7168, same bits);
// the two pairs of a row meet in LDS for the block max.
template <class T>
__device__ __forceinline__ void swiglu_quant_epilogue(v4f (&acc)[T::TM][T::TN], const QuantOut& qo,
                                                      int64_t m0, int64_t m_end, int64_t n0,
                                                      int64_t N, int wave, int wm0, int wn0,
                                                      int lane, const Stages<T>& st) {
    static_assert(T::WN == 64 && T::WAVES_N == 4 && T::BN == 256 && T::WAVES_M == 2,
                  "the gated epilogue runs on the 256 x 256 tile");
    const int lr = lane & 15, g = lane >> 4;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const bool is_up = (wn & 1) != 0;
    constexpr int HALF = T::TM / 2;                       // sub-tile rows each wave of a pair finishes
    constexpr int XFER = HALF * T::TN * 4;                // floats per lane handed to the partner
    static_assert(2 * 2 * XFER * 64 * 4 <= T::A_BYTES + T::B_BYTES, "hand-offs fit one stage");
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = bf16_round_f32(acc[i][j][r]);
    // The pair (g wave wn, u wave wn + 1) splits the rows: the g wave finishes sub-tile
    // rows 0 .. HALF-1, the u wave rows HALF .. TM-1.  Each hands the partner the values of
    // the rows the partner finishes: stage wm, column group wn >> 1 holds [g -> u | u -> g].
    float* x_gu = (float*)(wm == 0 ? st.p[0] : st.p[1]) + (wn >> 1) * 2 * XFER * 64;
    float* x_ug = x_gu + XFER * 64;
    // per-row maxima of the four waves of wave row wm: [4][WM], in that stage's scale area
    float* part = (float*)((wm == 0 ? st.p[0] : st.p[1]) + T::A_BYTES + T::B_BYTES);
    __syncthreads();                                               // every wave left the K loop
    if (is_up) {
#pragma unroll
        for (int i = 0; i < HALF; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) x_ug[((i * T::TN + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    } else {
#pragma unroll
        for (int i = 0; i < HALF; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x_gu[((i * T::TN + j) * 4 + r) * 64 + lane] = acc[HALF + i][j][r];
    }
    __syncthreads();
    // h = bf16(bf16(silu(g)) * u) for this wave's rows, kept in acc[HALF-offset rows]
    float pm[HALF];
    auto finish = [&](auto OFF_) __attribute__((always_inline)) {
        constexpr int OFF = decltype(OFF_)::value;       // 0: g wave, HALF: u wave
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            float m = 0.f;
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int x = ((i * T::TN + j) * 4 + r) * 64 + lane;
                    const float gv = OFF == 0 ? acc[i][j][r] : x_gu[x];
                    const float u = OFF == 0 ? x_ug[x] : acc[OFF + i][j][r];
                    const float sg = bf16_round_f32(gv / (1.0f + expf(-gv)));
                    const float h = bf16_round_f32(sg * u);
                    acc[OFF + i][j][r] = h;
                    m = fmaxf(m, fabsf(h));
                }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            pm[i] = m;
            if (g == 0) part[wn * T::WM + 16 * (OFF + i) + lr] = m;
        }
    };
    if (is_up) finish(StageId<HALF>{});
    else finish(StageId<0>{});
    __syncthreads();
    const int64_t nout = N / 2;
    const int64_t nbq = nout / kBlock;
    const int64_t h0 = n0 / 2 + (wn >> 1) * 64;                  // this pair's first h column
    // a 128-column block of h is the pair's 64 columns and the other pair's (wave wn ^ 2)
    auto encode = [&](auto OFF_) __attribute__((always_inline)) {
        constexpr int OFF = decltype(OFF_)::value;
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
            const float amax = fmaxf(pm[i], part[(wn ^ 2) * T::WM + 16 * (OFF + i) + lr]);
            const float s = fmaxf(amax, kAmaxFloor) / kE4m3Max;
            const float rcp = 1.0f / s;
            const int64_t row = m0 + wm0 + 16 * (OFF + i) + lr;
            if (row < m_end) {
                uint8_t* qrow = qo.q + row * nout + h0 + 4 * g;
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    const uint32_t codes = e4m3_encode4<true>(
                        quotient(acc[OFF + i][j][0], s, rcp), quotient(acc[OFF + i][j][1], s, rcp),
                        quotient(acc[OFF + i][j][2], s, rcp), quotient(acc[OFF + i][j][3], s, rcp));
                    *(uint32_t*)(qrow + 16 * j) = codes;
                }
                if (g == 0 && (wn >> 1) == 0) qo.qs[row * nbq + (n0 >> 8)] = s;
            }
        }
    };
    if (is_up) encode(StageId<HALF>{});
    else encode(StageId<0>{});
}

// kHwScale: every activation and weight scale is a power of two (the e8m0
// reading of scale_fmt), so the MFMA applies them itself (its per-row e8m0
// scale operands) and accumulates across K blocks with no fold.
// kStagedStore: interior bf16 tiles store through LDS (whole 128-byte row
// pieces); the grouped kernel leaves it off, since the extra epilogue path
// makes its heavy tile spill.
// kCls: 0 = every wave runs the same K loop; 1 and 2 = waves 0..3 and 4..7 of the
// split schedule (gemm_tile_big below).
template <class T, bool kGuard, int kEpi, bool kHwScale, bool kStagedStore, int kCls>
__device__ __forceinline__ void gemm_tile_body(const uint8_t* __restrict__ a,
                                              const float* __restrict__ as,
                                              const uint8_t* __restrict__ b,
                                              const float* __restrict__ bs,
                                              uint16_t* __restrict__ c, int64_t m0, int64_t m_end,
                                              int64_t n0, int64_t N, int64_t K,
                                              const Stages<T>& st, QuantOut qo = QuantOut{},
                                              PartialOut po = PartialOut{}) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / T::WAVES_N) * T::WM;
    const int wn0 = (wave % T::WAVES_N) * T::WN;
    const int64_t KB = K / kBlock;
    // the K blocks this tile multiplies: [K0, KE)
    const int64_t K0 = po.kb_lo, KE = po.kb_hi < 0 ? KB : po.kb_hi;
    const int64_t NBK = (N + kBlock - 1) / kBlock;
    const int64_t rows_a = (m_end - m0) < T::BM ? (m_end - m0) : T::BM;     // >= 1
    const int64_t rows_b = (N - n0) < T::BN ? (N - n0) : T::BN;            // >= 1

    // Buffer resources cover exactly the tile's valid rows (and the scale
    // rows), and every offset below stays inside them: rows past the end
    // read the last valid row and are never stored.
    const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a + m0 * K, (uint64_t)rows_a * K);
    const __amdgpu_buffer_rsrc_t rs_b = make_rsrc(b + n0 * K, (uint64_t)rows_b * K);
    const __amdgpu_buffer_rsrc_t rs_as = make_rsrc(as + m0 * KB, (uint64_t)rows_a * KB * 4);
    const __amdgpu_buffer_rsrc_t rs_bs =
        make_rsrc(bs, (uint64_t)((kEpi == kEpiSwiglu) ? (N + 63) / 64 : NBK) * KB * 4);

    // Direct-load sources (used by the loading waves, wave < LOADERS).
    // Instruction i of this wave fills LDS rows
    // r0 .. r0+7 (r0 = 8 * (wave * INSTR + i)); lane l writes physical chunk
    // l & 7 of row r0 + (l >> 3), which must hold logical chunk
    // (l & 7) ^ swz(row).  Offsets are relative to the tile's first row; the
    // K block enters as the scalar offset.
    const int lrow = lane >> 3;
    uint32_t a_off[T::A_INSTR], b_off[T::B_INSTR];
#pragma unroll
    for (int i = 0; i < T::A_INSTR; ++i) {
        int row = (wave * T::A_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        row = row < rows_a ? row : (int)rows_a - 1;
        a_off[i] = (uint32_t)(row * K) + chunk * 16;
    }
#pragma unroll
    for (int i = 0; i < T::B_INSTR; ++i) {
        int row = (wave * T::B_INSTR + i) * 8 + lrow;
        const int chunk = (lane & 7) ^ swz(row);
        row = row < rows_b ? row : (int)rows_b - 1;
        b_off[i] = (uint32_t)(row * K) + chunk * 16;
    }
    // row-scale slot p = t * SPITCH + i holds the activation scale of row
    // 16 i + t; other slots load row 0's scale (never read)
    uint32_t as_off;
    {
        const int p = wave * 64 + lane;
        const int t = p / T::SPITCH, i = p % T::SPITCH;
        int row = (t < 16 && i < T::BM / 16) ? 16 * i + t : 0;
        row = row < rows_a ? row : (int)rows_a - 1;
        as_off = (uint32_t)(row * KB * 4);
    }
    // weight-scale line: float l = scale of 128-column block (n0 / 128 + l)
    // weight scales: one per 128 weight rows, or per 64 rows for the
    // interleaved [w1; w3] weight (each 64-row group keeps its own block scale)
    constexpr int kSgShift = (kEpi == kEpiSwiglu) ? 6 : 7;
    const int64_t NBS = (kEpi == kEpiSwiglu) ? (N + 63) / 64 : NBK;
    uint32_t bs_off;
    {
        int64_t nb = (n0 >> kSgShift) + lane;
        nb = nb < NBS ? nb : NBS - 1;
        bs_off = (uint32_t)(nb * KB * 4);
    }

    // Split schedule.  Class 1 (waves 0..3) loads the A rows of block kb + 1 into
    // p[SF] after block kb's first sub-tile row; class 2 (waves 4..7) loads the weight
    // rows and scales of block kb + 2 into b[S] once every wave has read block kb's
    // (they are read into registers at the start of the block), after a second
    // barrier.  So the weight rows get two blocks of lead with two stages, and each
    // class is held by the vector-memory path for half a block's loads.  Offsets are
    // the instruction's parity (the swizzle) with the eight-row steps in the scalar
    // offset; rows past the tile read as zeros.
    static_assert(kCls == 0 || (T::NSTAGE == 2 && T::WAVES == 8 && T::LOADERS == 4 && !kHwScale &&
                                T::A_INSTR % 2 == 0 && T::B_INSTR % 2 == 0),
                  "the split schedule runs on the two-stage eight-wave tile");
    constexpr int kRowsBeforeSync = 5;                // class 2: sub-tile rows before barrier 2
    constexpr int kLoadsB = T::B_INSTR + 2;           // class 2: loads per wave per block
    const uint32_t K32 = (uint32_t)K;
    uint32_t v_par[2];
    v_par[0] = (uint32_t)lrow * K32 + (uint32_t)(((lane & 7) ^ lrow) << 4);
    v_par[1] = (uint32_t)lrow * K32 + (uint32_t)(((lane & 7) ^ lrow ^ 1) << 4);
    // class 2 wave cw's two scale loads: row-scale instruction 2 cw + h while there is
    // one (S_INSTR of them), else the weight-scale line; wave 7 repeats instruction 4
    // and the line, so every wave counts the same loads
    const int cw = wave - 4;
    uint32_t sc_off[2], sc_lds[2];
    bool sc_row[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int idx = 2 * cw + h;
        if (idx == 6) idx = T::S_INSTR - 1;
        sc_row[h] = idx < T::S_INSTR;
        const int pq = (sc_row[h] ? idx : 0) * 64 + lane;
        const int t = pq / T::SPITCH, i = pq % T::SPITCH;
        int row = (t < 16 && i < T::BM / 16) ? 16 * i + t : 0;
        row = row < rows_a ? row : (int)rows_a - 1;
        sc_off[h] = sc_row[h] ? (uint32_t)(row * KB * 4) : bs_off;
        sc_lds[h] = sc_row[h] ? (uint32_t)(T::B_BYTES + idx * 256) : (uint32_t)(T::B_BYTES + T::SB_OFF);
    }
    auto issue_a = [&](int64_t kb, uint8_t* base) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)(kb * kBlock);
#pragma unroll
        for (int i = 0; i < T::A_INSTR; ++i) {
            const uint32_t r0 = (uint32_t)((wave * T::A_INSTR + i) * 8);
            buf_lds16(rs_a, v_par[i & 1], ko + r0 * K32, base + (wave * T::A_INSTR + i) * 1024);
        }
    };
    auto issue_b = [&](int64_t kb, uint8_t* base) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)(kb * kBlock);
#pragma unroll
        for (int i = 0; i < T::B_INSTR; ++i) {
            const uint32_t r0 = (uint32_t)((cw * T::B_INSTR + i) * 8);
            buf_lds16(rs_b, v_par[i & 1], ko + r0 * K32, base + (cw * T::B_INSTR + i) * 1024);
        }
        const uint32_t so = (uint32_t)(kb * 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (sc_row[h]) buf_lds4(rs_as, sc_off[h], so, base + sc_lds[h]);
            else buf_lds4(rs_bs, sc_off[h], so, base + sc_lds[h]);
        }
    };

    auto issue = [&](int64_t kb, uint8_t* base) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)(kb * kBlock);
        if (T::LOADERS == T::WAVES || wave < T::LOADERS) {
#pragma unroll
            for (int i = 0; i < T::A_INSTR; ++i)
                buf_lds16(rs_a, a_off[i], ko, base + (wave * T::A_INSTR + i) * 1024);
#pragma unroll
            for (int i = 0; i < T::B_INSTR; ++i)
                buf_lds16(rs_b, b_off[i], ko, base + T::A_BYTES + (wave * T::B_INSTR + i) * 1024);
        }
        const uint32_t so = (uint32_t)(kb * 4);
        if (T::NSTAGE > 2 || wave < T::S_INSTR)
            buf_lds4(rs_as, as_off, so, base + T::A_BYTES + T::B_BYTES + wave * 256);
        if (T::NSTAGE > 2 || wave == 0)
            buf_lds4(rs_bs, bs_off, so, base + T::A_BYTES + T::B_BYTES + T::SB_OFF);
    };
    // load q of a stage, in issue()'s order: A rows, B rows, row scales, weight scales
    auto issue_one = [&](int q, int64_t kb, uint8_t* base) __attribute__((always_inline)) {
        const uint32_t ko = (uint32_t)(kb * kBlock);
        const uint32_t so = (uint32_t)(kb * 4);
        if (q < T::A_INSTR)
            buf_lds16(rs_a, a_off[q], ko, base + (wave * T::A_INSTR + q) * 1024);
        else if (q < T::A_INSTR + T::B_INSTR)
            buf_lds16(rs_b, b_off[q - T::A_INSTR], ko,
                      base + T::A_BYTES + (wave * T::B_INSTR + q - T::A_INSTR) * 1024);
        else if (q == T::A_INSTR + T::B_INSTR)
            buf_lds4(rs_as, as_off, so, base + T::A_BYTES + T::B_BYTES + wave * 256);
        else
            buf_lds4(rs_bs, bs_off, so, base + T::A_BYTES + T::B_BYTES + T::SB_OFF);
    };
    // With two stages the next block's loads go out right after the barrier
    // (they get one block of lead); with three or more they are spread over
    // the first rows' MFMAs of the full-tile loop, so no wave stalls on a long
    // burst of load issues while its MFMAs wait.
    constexpr bool kSpread = T::NSTAGE > 2;

    v4f acc[T::TM][T::TN];
    // The unguarded fold loop folds the last sub-tile row of block kb during
    // the first row's MFMAs of block kb + 1 (so no wave ends a block with folds
    // that no MFMA hides): prev holds that row's block products, sc_last its
    // scale.  Each sum still takes its block terms in order, so the results
    // are the same bits.
    v4f prev[T::TN];
    float sc_last = 0.f;
#pragma unroll
    for (int j = 0; j < T::TN; ++j) prev[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // a workgroup that walks several tiles must not refill a stage that a
    // slower wave still reads for the previous tile, and every wave's loads
    // of the previous tile have landed (all waves write the weight-scale line)
    wait_vmcnt<0>();
    barrier_lds();
    int tm_valid = T::TM;
    if (kGuard) {
        const int64_t rows = m_end - (m0 + wm0);
        tm_valid = rows <= 0 ? 0 : (rows >= 16 * T::TM ? T::TM : (int)((rows + 15) / 16));
        tm_valid = __builtin_amdgcn_readfirstlane(tm_valid);
    }

    // Waves w and w + 4 share a SIMD.  Left alone, the scheduler favours the
    // older of the two, which finishes its block early and waits at the barrier
    // while the other runs alone; raising waves 4..7 one priority level keeps
    // each pair even (2-6% faster on the eight-wave tiles, same bits; raising
    // waves 0..3 instead, or alternating by block, measured no better).
    // In the split schedule class 1 runs one level up instead: it is the class whose
    // multiplies end the block (measured 0.5-1% faster than raising class 2).
    if (kCls != 0 ? kCls == 1 : (T::WAVES == 8 && wave >= 4)) __builtin_amdgcn_s_setprio(1);

    // prologue: K blocks 0 .. NSTAGE-2 in flight, block s in stage s (split schedule:
    // the A rows of block 0 and the weight rows of blocks 0 and 1)
    if constexpr (kCls == 1) {
        issue_a(K0, st.p[0]);
    } else if constexpr (kCls == 2) {
        issue_b(K0, st.b[0]);
        issue_b(K0 + 1 < KE ? K0 + 1 : K0, st.b[1]);
    } else {
        issue(K0, st.p[0]);
    }
    if (kCls == 0 && T::NSTAGE > 2 && K0 + 1 < KE) issue(K0 + 1, st.p[1]);
    if (T::NSTAGE > 3 && K0 + 2 < KE) issue(K0 + 2, st.p[2]);

    const int lr = lane & 15;
    const int lk = (lane >> 4) * 2;
    const int off0 = ((lk ^ swz(lr)) << 4);
    const int off1 = (((lk + 1) ^ swz(lr)) << 4);
    const int sread = lr * T::SPITCH + wm0 / 16;
    const int sb_slot = wn0 >> kSgShift;               // this wave's weight-scale float

    // One K block from stage S; block kb + NSTAGE - 1 goes to the stage that
    // block kb - 1 used.
    auto step = [&](int64_t kb, auto S_) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        constexpr int SF = (S + T::NSTAGE - 1) % T::NSTAGE;
        // this wave's loads of block kb are done once at most the loads of
        // blocks kb+1 .. kb+NSTAGE-2 are outstanding (loads complete in issue
        // order); the barrier then makes every wave's loads visible and
        // guarantees stage SF (block kb - 1) is no longer being read
        // (split schedule: class 1 waits for its A rows of block kb, class 2 for its
        // weight rows of block kb while those of kb + 1 may still be in flight)
        if constexpr (kCls == 2) {
            wait_vmcnt<kLoadsB>();
        } else if constexpr (kCls == 1) {
            wait_vmcnt<0>();
        } else {
            if (kb + T::NSTAGE - 2 < KE)
                wait_vmcnt<T::LOADS_PER_STAGE * (T::NSTAGE - 2)>();
            else
                wait_vmcnt<0>();
        }
        barrier_lds();
        const bool more = kb + T::NSTAGE - 1 < KE;
        // (the spread issue lives in the fold loop; the power-of-two-scale loop issues here)
        if (kCls == 0 && (!kSpread || kHwScale) && more) issue(kb + T::NSTAGE - 1, st.p[SF]);

        const uint8_t* As = st.p[S];
        const uint8_t* Bs = kCls != 0 ? st.b[S] : As + T::A_BYTES;
        const float* Ss = (const float*)(Bs + T::B_BYTES);
        const float* Sb = (const float*)(Bs + T::B_BYTES + T::SB_OFF);
        if constexpr (kHwScale) {
            // scale operands: the weight first (uniform over the wave's columns), the
            // activation second (lane l: row 16 i + (l & 15)); e8m0 byte = fp32 exponent
            v8i fb[T::TN];
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const uint8_t* q = Bs + (wn0 + 16 * j + lr) * kBlock;
                fb[j] = frag_from(*(const uint4*)(q + off0), *(const uint4*)(q + off1));
            }
            const int eb = (int)(__float_as_uint(Sb[sb_slot]) >> 23);
            int ea[T::TM];
#pragma unroll
            for (int i = 0; i < T::TM; i += 4) {
                const v4f s4 = *(const v4f*)(Ss + sread + i);
                ea[i] = (int)(__float_as_uint(s4[0]) >> 23);
                ea[i + 1] = (int)(__float_as_uint(s4[1]) >> 23);
                ea[i + 2] = (int)(__float_as_uint(s4[2]) >> 23);
                ea[i + 3] = (int)(__float_as_uint(s4[3]) >> 23);
            }
            v8i fa_nxt;
            {
                const uint8_t* r = As + (wm0 + lr) * kBlock;
                fa_nxt = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i) {
                const v8i fa = fa_nxt;
                if (i + 1 < T::TM) {
                    const uint8_t* r = As + (wm0 + 16 * (i + 1) + lr) * kBlock;
                    fa_nxt = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
                }
                if (!kGuard || i < tm_valid) {
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            fb[j], fa, acc[i][j], 0, 0, 0, eb, 0, ea[i]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // The K block as a fixed sequence of small scheduling regions
            // (sched_barrier keeps the compiler from reordering across them):
            // a wave starts multiplying once A row 0 and B fragment 0 are in
            // registers; each further B fragment is read during the previous
            // MFMA; the scales arrive with the last MFMA of row 0; then every
            // sub-tile row issues its TN MFMAs interleaved with the folds of
            // the previous row while the next A row is read.
            v8i fb[T::TN];
            v8i fa_cur, fa_nxt;
            v4f cur_p[T::TN];
            float sc[T::TM];
            {
                const uint8_t* r = As + (wm0 + lr) * kBlock;
                fa_cur = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
                const uint8_t* q = Bs + (wn0 + lr) * kBlock;
                fb[0] = frag_from(*(const uint4*)(q + off0), *(const uint4*)(q + off1));
            }
            __builtin_amdgcn_sched_barrier(0);
            v4f s4[T::TM / 4];
            float sbv = 0.f;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                if (j + 1 < T::TN) {
                    const uint8_t* q = Bs + (wn0 + 16 * (j + 1) + lr) * kBlock;
                    fb[j + 1] = frag_from(*(const uint4*)(q + off0), *(const uint4*)(q + off1));
                } else {
#pragma unroll
                    for (int i = 0; i < T::TM; i += 4) s4[i / 4] = *(const v4f*)(Ss + sread + i);
                    sbv = Sb[sb_slot];
                }
                cur_p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fb[j], fa_cur, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                acc[T::TM - 1][j] = prev[j] * sc_last + acc[T::TM - 1][j];
                __builtin_amdgcn_sched_barrier(0);
            }
            {
                const uint8_t* r = As + (wm0 + 16 + lr) * kBlock;
                fa_nxt = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
            }
#pragma unroll
            for (int i = 0; i < T::TM; i += 4) {
                sc[i] = s4[i / 4][0] * sbv; sc[i + 1] = s4[i / 4][1] * sbv;
                sc[i + 2] = s4[i / 4][2] * sbv; sc[i + 3] = s4[i / 4][3] * sbv;
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j) prev[j] = cur_p[j];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 1; i < T::TM; ++i) {
                if constexpr (kCls != 0) {
                    if (i == (kCls == 1 ? 1 : kRowsBeforeSync)) {
                        if constexpr (kCls == 1) {
                            if (more) issue_a(kb + 1, st.p[SF]);
                        }
                        // barrier 2: every wave has read block kb's weight rows and scales
                        barrier_lds();
                        // (past the last block the last one is loaded again, never read)
                        if constexpr (kCls == 2) issue_b(kb + 2 < KE ? kb + 2 : KE - 1, st.b[S]);
                    }
                }
                if (kSpread && more) {
                    constexpr int NQ = T::LOADS_PER_STAGE;
                    const int q0 = 2 * (i - 1);
                    if (q0 < NQ) issue_one(q0, kb + T::NSTAGE - 1, st.p[SF]);
                    if (q0 + 1 < NQ) issue_one(q0 + 1, kb + T::NSTAGE - 1, st.p[SF]);
                    if (i == T::TM - 1) {
#pragma unroll
                        for (int q = q0 + 2; q < NQ; ++q) issue_one(q, kb + T::NSTAGE - 1, st.p[SF]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                fa_cur = fa_nxt;
                if (i + 1 < T::TM) {
                    const uint8_t* r = As + (wm0 + 16 * (i + 1) + lr) * kBlock;
                    fa_nxt = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
                }
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    cur_p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fb[j], fa_cur, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    acc[i - 1][j] = prev[j] * sc[i - 1] + acc[i - 1][j];
                }
#pragma unroll
                for (int j = 0; j < T::TN; ++j) prev[j] = cur_p[j];
                // per MFMA four folds of the previous row; the next row's A reads go out
                // after the first MFMA (about 1% faster than before it)
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (j == 0 && i + 1 < T::TM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sc_last = sc[T::TM - 1];
        }
    };

    // (the split schedule needs an even block count: class 2 runs the second step
    // unconditionally, which keeps the compiler's wait for its in-flight weight
    // loads precise across the loop's back edge)
    for (int64_t kb0 = K0; kb0 < KE; kb0 += T::NSTAGE) {
        step(kb0, StageId<0>{});
        if (kCls == 2 || kb0 + 1 < KE) step(kb0 + 1, StageId<1>{});
        if constexpr (T::NSTAGE > 2) {
            if (kb0 + 2 < KE) step(kb0 + 2, StageId<2>{});
        }
        if constexpr (T::NSTAGE > 3) {
            if (kb0 + 3 < KE) step(kb0 + 3, StageId<3>{});
        }
    }

    if constexpr (kCls != 0) wait_vmcnt<0>();      // class 2's reloads of the last block
    // the last block's last row (the fold loop carries it into the next block)
    if constexpr (!kHwScale) {
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[T::TM - 1][j] = prev[j] * sc_last + acc[T::TM - 1][j];
    }
    // epilogue: lane holds row m0 + wm0 + 16 i + lr, columns n0 + wn0 + 16 j + 4 (lane >> 4) + 0..3
    if constexpr (kEpi == kEpiQuant) {
        uint8_t* cbuf = kCls != 0 ? (wave < 4 ? st.p[1] : st.b[1]) + (wave & 3) * (T::WM * 64)
                                  : st.p[1] + wave * (T::WM * 64);
        quant_epilogue<T>(acc, qo, m0, m_end, n0, N, wave, wm0, wn0, lane, st.p[0], cbuf);
        return;
    }
    if constexpr (kEpi == kEpiSwiglu) {
        swiglu_quant_epilogue<T>(acc, qo, m0, m_end, n0, N, wave, wm0, wn0, lane, st);
        return;
    }
    if constexpr (kEpi == kEpiF32) {
        const int cq = 4 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            const int64_t row = m0 + wm0 + 16 * i + lr;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int64_t col = n0 + wn0 + 16 * j + cq;
                if (row < m_end && col + 3 < N)
                    *(v4f*)(po.ws + row * po.ldw + (col - po.n_base)) = acc[i][j];
            }
        }
        return;
    }
    const int cq = 4 * (lane >> 4);
    const bool interior = (m0 + T::BM <= m_end) && (n0 + T::BN <= N);
    // 8-byte stores wherever the tile's columns are whole; rows tested one by one
    const bool vec = (n0 + T::BN <= N) && (N % 4 == 0) && (((uintptr_t)c & 7u) == 0);
    // rows per pass of the staged store: 64 where every wave's 8 KB fits one stage, else 32
    constexpr int kRP = T::WAVES * 64 * 128 <= T::STAGE ? 64 : 32;
    constexpr int kSub = kRP / 16;                          // sub-tile rows per pass
    if constexpr (kStagedStore && T::WN == 64 && T::TM % kSub == 0 &&
                  T::WAVES * kRP * 128 <= T::STAGE) {
        // After a barrier (no loads are in flight after the last K block) the
        // first stage is free.  Each wave turns kRP of its rows at a time into
        // bf16 rows of 128 bytes there (16-byte chunks XOR-swizzled by row),
        // then stores whole 128-byte row pieces, 16 bytes per lane.
        if (interior && vec && (N % 8 == 0) && (((uintptr_t)c & 15u) == 0)) {
            __syncthreads();                      // every wave is past its last LDS read
            uint8_t* buf = kCls != 0 ? (wave < 4 ? st.p[0] : st.b[0]) + (wave & 3) * (kRP * 128)
                                     : st.p[0] + wave * (kRP * 128);
#pragma unroll
            for (int h = 0; h < T::TM / kSub; ++h) {
#pragma unroll
                for (int i = 0; i < kSub; ++i) {
                    const int r = 16 * i + lr;
#pragma unroll
                    for (int j = 0; j < T::TN; ++j) {
                        const int byte = (16 * j + cq) * 2;
                        uint2 v;
                        v.x = pack_bf16x2(acc[kSub * h + i][j][0], acc[kSub * h + i][j][1]);
                        v.y = pack_bf16x2(acc[kSub * h + i][j][2], acc[kSub * h + i][j][3]);
                        *(uint2*)(buf + r * 128 + ((((byte >> 4) ^ (r & 7))) << 4) + (byte & 15)) = v;
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
            if (kGuard && m0 + wm0 + 16 * i + lr >= m_end) continue;
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

// One large tile.  kSplit: the split schedule (gemm_tile_body), for the two-stage
// eight-wave tile on whole tiles (rows m0 .. m0 + BM - 1 all valid) with an even
// K-block count; the stages then hold the A rows in st.p[s] and the weight rows and
// scales in st.b[s].  Against every wave issuing its share right after one barrier per
// block (waves 0..3 all of it), the waves of each SIMD pair are held by the
// vector-memory path half as long and the weight rows land a block earlier:
// per-block cycles 2925 -> 2780, the raised waves' barrier wait 1473 -> 465
// (8192 x 18432 x 7168, same bits).
template <class T, bool kGuard, int kEpi = kEpiBf16, bool kHwScale = false,
          bool kStagedStore = true, bool kSplit = false>
__device__ __forceinline__ void gemm_tile_big(const uint8_t* __restrict__ a,
                                              const float* __restrict__ as,
                                              const uint8_t* __restrict__ b,
                                              const float* __restrict__ bs,
                                              uint16_t* __restrict__ c, int64_t m0, int64_t m_end,
                                              int64_t n0, int64_t N, int64_t K,
                                              const Stages<T>& st, QuantOut qo = QuantOut{},
                                              PartialOut po = PartialOut{}) {
    if constexpr (kSplit) {
        static_assert(!kGuard, "the split schedule runs whole tiles");
        if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
            gemm_tile_body<T, false, kEpi, kHwScale, kStagedStore, 1>(a, as, b, bs, c, m0, m_end,
                                                                      n0, N, K, st, qo, po);
        else
            gemm_tile_body<T, false, kEpi, kHwScale, kStagedStore, 2>(a, as, b, bs, c, m0, m_end,
                                                                      n0, N, K, st, qo, po);
    } else {
        gemm_tile_body<T, kGuard, kEpi, kHwScale, kStagedStore, 0>(a, as, b, bs, c, m0, m_end, n0,
                                                                   N, K, st, qo, po);
    }
}

// The stage arrays of a large-tile kernel (unused ones are 16 bytes).
#define BIG_TILE_STAGES(T, st)                                                            \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_0[T::STAGE];                    \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_1[T::STAGE];                    \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_2[T::NSTAGE > 2 ? T::STAGE : 16]; \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_3[T::NSTAGE > 3 ? T::STAGE : 16]; \
    const Stages<T> st = {{st##_0, st##_1, st##_2, st##_3}, {nullptr, nullptr, nullptr, nullptr}}

// The split schedule's arrays: A rows, and weight rows with scales, per stage.
#define BIG_TILE_SPLIT_STAGES(T, st)                                                      \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_a0[T::A_BYTES];                 \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_b0[T::B_BYTES + T::S_BYTES];    \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_a1[T::A_BYTES];                 \
    __shared__ __attribute__((aligned(1024))) uint8_t st##_b1[T::B_BYTES + T::S_BYTES];    \
    const Stages<T> st = {{st##_a0, st##_a1, nullptr, nullptr}, {st##_b0, st##_b1, nullptr, nullptr}}

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

// kSplit: the split schedule; the host launches it only for whole M tiles and an even
// K-block count.
template <class T, bool kSplit = false>
__global__ __launch_bounds__(T::THREADS, T::OCC) void gemm_big_kernel(const uint8_t* __restrict__ a,
                                                                 const float* __restrict__ as,
                                                                 const uint8_t* __restrict__ b,
                                                                 const float* __restrict__ bs,
                                                                 uint16_t* __restrict__ c,
                                                                 int64_t M, int64_t N, int64_t K,
                                                                 int mt, int nt) {
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM;
    if constexpr (kSplit) {
        BIG_TILE_SPLIT_STAGES(T, lds);
        gemm_tile_big<T, false, kEpiBf16, false, true, true>(a, as, b, bs, c, m0, M,
                                                            (int64_t)tn * T::BN, N, K, lds);
    } else {
        BIG_TILE_STAGES(T, lds);
        if (m0 + T::BM <= M)
            gemm_tile_big<T, false>(a, as, b, bs, c, m0, M, (int64_t)tn * T::BN, N, K, lds);
        else
            gemm_tile_big<T, true>(a, as, b, bs, c, m0, M, (int64_t)tn * T::BN, N, K, lds);
    }
}

// The last, partly filled round of a large GEMM ("tail"): columns
// [n1, N) in full 256-column tiles, each tile's K blocks split in `splits`
// runs of kb_per blocks, so twice as many workgroups fill the round.  Split s
// writes its fp32 partial sums to ws[s][M][N - n1]; tail_reduce_kernel adds
// them in split order.  Workgroup id = s * tiles + tile, the tiles of one
// split laid out over the XCDs as in gemm_big_kernel.  kHw: the power-of-two
// scale GEMM (scales applied by the MFMA).
template <class T, bool kHw = false, bool kSplit = false>
__global__ __launch_bounds__(T::THREADS, 1) void gemm_tail_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, float* __restrict__ ws, int64_t M, int64_t N, int64_t K, int mt,
    int nt_tail, int64_t n1, int64_t kb_per) {
    const int tiles = mt * nt_tail;
    const int split = blockIdx.x / tiles;
    int tm, tn;
    tile_of(blockIdx.x - split * tiles, tiles, mt, nt_tail, tm, tn);
    const int64_t KB = K / kBlock;
    PartialOut po;
    po.kb_lo = split * kb_per;
    po.kb_hi = po.kb_lo + kb_per < KB ? po.kb_lo + kb_per : KB;
    po.ldw = N - n1;
    po.ws = ws + (int64_t)split * M * po.ldw;
    po.n_base = n1;
    if constexpr (kSplit) {
        // (the host launches this form when both K runs hold an even block count)
        BIG_TILE_SPLIT_STAGES(T, lds);
        gemm_tile_big<T, false, kEpiF32, false, true, true>(a, as, b, bs, nullptr, (int64_t)tm * T::BM,
                                                           M, n1 + (int64_t)tn * T::BN, N, K, lds,
                                                           QuantOut{}, po);
    } else {
        BIG_TILE_STAGES(T, lds);
        gemm_tile_big<T, false, kEpiF32, kHw>(a, as, b, bs, nullptr, (int64_t)tm * T::BM, M,
                                              n1 + (int64_t)tn * T::BN, N, K, lds, QuantOut{}, po);
    }
}

// The GEMM with power-of-two scales applied by the MFMA (kHwScale).
template <class T>
__global__ __launch_bounds__(T::THREADS, T::OCC) void gemm_ue8m0_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, uint16_t* __restrict__ c, int64_t M, int64_t N, int64_t K, int mt,
    int nt) {
    BIG_TILE_STAGES(T, lds);
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM;
    if (m0 + T::BM <= M)
        gemm_tile_big<T, false, kEpiBf16, true>(a, as, b, bs, c, m0, M, (int64_t)tn * T::BN, N, K, lds);
    else
        gemm_tile_big<T, true, kEpiBf16, true>(a, as, b, bs, c, m0, M, (int64_t)tn * T::BN, N, K, lds);
}

// The same GEMM with act_quant of its output (kEpi = kEpiQuant), or of the
// gated activation of an interleaved [w1; w3] product (kEpiSwiglu), fused
// into the epilogue.
template <class T, int kEpi, bool kSplit = false>
__global__ __launch_bounds__(T::THREADS, T::OCC) void gemm_quant_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, uint8_t* __restrict__ q, float* __restrict__ qs, int64_t M,
    int64_t N, int64_t K, int mt, int nt) {
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, mt, nt, tm, tn);
    const int64_t m0 = (int64_t)tm * T::BM;
    const QuantOut qo{q, qs};
    if constexpr (kSplit) {
        static_assert(kEpi == kEpiQuant, "the split schedule serves the act_quant epilogue");
        BIG_TILE_SPLIT_STAGES(T, lds);
        gemm_tile_big<T, false, kEpi, false, true, true>(a, as, b, bs, nullptr, m0, M,
                                                        (int64_t)tn * T::BN, N, K, lds, qo);
    } else {
        BIG_TILE_STAGES(T, lds);
        if (m0 + T::BM <= M)
            gemm_tile_big<T, false, kEpi>(a, as, b, bs, nullptr, m0, M, (int64_t)tn * T::BN, N, K, lds, qo);
        else
            gemm_tile_big<T, true, kEpi>(a, as, b, bs, nullptr, m0, M, (int64_t)tn * T::BN, N, K, lds, qo);
    }
}

// Split-K kernel for skinny problems (those split_plan splits).  A workgroup owns a 64 x 64
// output tile and a run of at most SK_DEEP_KB K blocks; it issues every
// direct-to-LDS load of that run at once (one memory latency per workgroup
// instead of one per K block), waits once, then multiplies.  Four waves of
// 32 x 32 (2 x 2 sub-tiles), MFMA operands weight-first as in the large-tile
// kernel (a lane owns one output row and four consecutive columns), scales
// read straight from global memory.  The fp32 partial sums of split s go to
// ws[s][M][N]; split_reduce_kernel adds the splits in index order.
constexpr int SK_MAX_KB = 4;          // 64 KB of LDS: two workgroups per CU
constexpr int SK_DEEP_KB = 8;         // 128 KB of LDS: one workgroup per CU

__global__ __launch_bounds__(256) void gemm_skinny_kernel(const uint8_t* __restrict__ a,
                                                          const float* __restrict__ as,
                                                          const uint8_t* __restrict__ b,
                                                          const float* __restrict__ bs,
                                                          float* __restrict__ ws, int64_t M,
                                                          int64_t N, int64_t K, int mt,
                                                          int kb_per) {
    constexpr int BM = 64, BN = 64, BLK = (BM + BN) * kBlock;       // 16 KB per K block
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];  // kb_per * BLK bytes
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tm = blockIdx.x % mt, tn = blockIdx.x / mt;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int64_t KB = K / kBlock;
    const int64_t kb0 = (int64_t)blockIdx.y * kb_per;
    const int nkb = (int)((kb0 + kb_per < KB ? kb0 + kb_per : KB) - kb0);
    const int64_t NBK = (N + kBlock - 1) / kBlock;

    // loads: per K block, 16 instructions of 1 KB (8 for A rows, 8 for B rows),
    // wave w issues instructions w, w+4, w+8, w+12
    const int lrow = lane >> 3;
    for (int kb = 0; kb < nkb; ++kb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ins = wave + 4 * q;              // 0..15
            const bool is_a = ins < 8;
            const int row = (is_a ? ins : ins - 8) * 8 + lrow;
            const int chunk = (lane & 7) ^ swz(row);
            const uint8_t* src;
            if (is_a) {
                int64_t g = m0 + row;
                g = g < M ? g : M - 1;
                src = a + g * K;
            } else {
                int64_t g = n0 + row;
                g = g < N ? g : N - 1;
                src = b + g * K;
            }
            load_lds16(src + (kb0 + kb) * kBlock + chunk * 16, lds + kb * BLK + ins * 1024);
        }
    }
    const int wm0 = (wave >> 1) * 32, wn0 = (wave & 1) * 32;
    const int lr = lane & 15;
    // activation scales of this lane's two rows and the wave's weight scale, per K block
    int64_t r0 = m0 + wm0 + lr, r1 = r0 + 16;
    r0 = r0 < M ? r0 : M - 1;
    r1 = r1 < M ? r1 : M - 1;
    int64_t nb = (n0 + wn0) >> 7;
    nb = nb < NBK ? nb : NBK - 1;
    wait_vmcnt<0>();
    barrier_lds();

    const int lk = (lane >> 4) * 2;
    const int off0 = ((lk ^ swz(lr)) << 4);
    const int off1 = (((lk + 1) ^ swz(lr)) << 4);
    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < nkb; ++kb) {
        const uint8_t* As = lds + kb * BLK;
        const uint8_t* Bs = As + BM * kBlock;
        v8i fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint8_t* r = As + (wm0 + 16 * i + lr) * kBlock;
            fa[i] = frag_from(*(const uint4*)(r + off0), *(const uint4*)(r + off1));
            const uint8_t* q = Bs + (wn0 + 16 * i + lr) * kBlock;
            fb[i] = frag_from(*(const uint4*)(q + off0), *(const uint4*)(q + off1));
        }
        const int64_t k = kb0 + kb;
        const float sbv = bs[nb * KB + k];
        const float sc0 = as[r0 * KB + k] * sbv, sc1 = as[r1 * KB + k] * sbv;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v4f p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fb[j], fa[0], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            const v4f p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fb[j], fa[1], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            acc[0][j] = p0 * sc0 + acc[0][j];
            acc[1][j] = p1 * sc1 + acc[1][j];
        }
    }
    float* part = ws + (int64_t)blockIdx.y * M * N;
    const int cq = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t row = m0 + wm0 + 16 * i + lr;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn0 + 16 * j + cq;
            float* dst = part + row * N + col;
            if (col + 3 < N && (N % 4 == 0)) {
                *(v4f*)dst = acc[i][j];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (col + r < N) dst[r] = acc[i][j][r];
            }
        }
    }
}


// Split-K plan for skinny problems: M <= 64, or M <= 256 when the problem
// makes at most 32 tiles of 128 x 128 (an eighth of the chip's CUs; those
// ran one round of mostly idle CUs: 128 x 2048 x 7168 took 16.5 us split
// against 33.4 us whole, 256 x 1536 x 7168 24.1 against 33.6, 100 x 4096 x
// 7168 26.7 against 38.7, while 256 x 4096 x 7168 was slower split).  Deep
// splits of up to 8 K blocks when that makes at most 512 workgroups (the
// decode-sized shapes: fewer partial sums to write and add, measured 10-16%
// faster on 64 x 1536 x 7168, 64 x 7168 x 2048 and 32 x 2048 x 7168);
// otherwise enough (tile, split) pairs for about 384 workgroups, at most 4
// and at least 2 K blocks per split (wide or long-K shapes, e.g.
// 64 x 18432 x 7168 and 16 x 7168 x 18432, were faster that way).
// Host-only arithmetic, so bfp8_gemm_workspace_size needs no device.
struct SplitPlan {
    int splits, kb_per;
};

static SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
    SplitPlan p{1, (int)(K / kBlock)};
    if (M > 256 || (M > 64 && ((M + 127) / 128) * ((N + 127) / 128) > 32)) return p;
    const int64_t tiles = ((M + 63) / 64) * ((N + 63) / 64);
    const int64_t KB = K / kBlock;
    if (KB > SK_DEEP_KB) {
        const int64_t splits = (KB + SK_DEEP_KB - 1) / SK_DEEP_KB;
        if (tiles * splits <= 512) {
            p.kb_per = (int)((KB + splits - 1) / splits);
            p.splits = (int)splits;
            return p;
        }
    }
    int64_t want = (384 + tiles - 1) / tiles;
    if (want > KB / 2) want = KB / 2;
    if (want < 2) return p;
    int64_t kb_per = (KB + want - 1) / want;
    kb_per = kb_per < SK_MAX_KB ? kb_per : SK_MAX_KB;
    p.kb_per = (int)kb_per;
    p.splits = (int)((KB + kb_per - 1) / kb_per);
    return p;
}

// Tail plan for large GEMMs on 256 x 256 tiles: when the tiles fill a few
// whole rounds of the chip's 256 CUs and a last round at most half full, and
// that last round is whole columns of tiles (rem = mt * nt_tail), the tail
// columns run as two K halves (twice the workgroups) into an fp32 workspace,
// then one reduction.  Measured on 8192 x 7168 x 18432 (3.5 rounds): the half
// round cost 0.79 of a full round before.  Only for K of 80 blocks and more:
// on 8192 x 7168 x K the split tail won at K = 12288 and 18432 (915.9 against
// 931.8 us at 18432) and lost from K = 7168 down (134 against 115 us at
// 2048), where the partial sums' write and reduction outweigh the half round.
// Host-only arithmetic, planned for 256 CUs, so bfp8_gemm_workspace_size
// needs no device.
TailPlan tail_plan(int64_t M, int64_t N, int64_t K) {
    TailPlan p;
    constexpr int64_t kCUs = 256;
    if (M <= 128 || M % 256 != 0 || N % 256 != 0) return p;
    const int64_t mt = M / 256, nt = N / 256, tiles = mt * nt, KB = K / kBlock;
    const int64_t rem = tiles % kCUs;
    if (tiles < kCUs || rem == 0 || rem % mt != 0 || 2 * rem > kCUs || KB < 80) return p;
    p.nt_tail = (int)(rem / mt);
    p.nt_main = (int)(nt - p.nt_tail);
    p.splits = 2;
    p.kb_per = (KB + 1) / 2;
    return p;
}

size_t tail_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const TailPlan p = tail_plan(M, N, K);
    if (p.splits == 0) return 0;
    return (size_t)p.splits * (size_t)M * (size_t)p.nt_tail * 256 * sizeof(float);
}

static size_t round256(size_t v) { return (v + 255) / 256 * 256; }

// The FP8 branch of linear(): act_quant of x into the workspace, then the
// GEMM, split over K (partials after the codes) where split_plan splits.
// A single kernel that also reduces the splits (the last workgroup of a tile
// adding them) was slower on this chip: publishing partials across XCDs costs
// an L2 write-back per workgroup and an invalidate per tile, more than the two
// extra launches.
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    return round256((size_t)M * K) + round256((size_t)M * (K / kBlock) * 4) +
           round256(gemm_workspace_bytes(M, N, K));
}

hipError_t launch_linear_fp8(const void* x, const void* b, const float* bs, void* c, int64_t M,
                             int64_t N, int64_t K, void* workspace, hipStream_t stream) {
    uint8_t* q = (uint8_t*)workspace;
    float* qs = (float*)(q + round256((size_t)M * K));
    uint8_t* part = (uint8_t*)qs + round256((size_t)M * (K / kBlock) * 4);
    hipError_t e = launch_act_quant(x, q, qs, M, K, stream);
    if (e != hipSuccess) return e;
    return launch_gemm(q, qs, b, bs, c, M, N, K, part, gemm_workspace_bytes(M, N, K), stream);
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitPlan p = split_plan(M, N, K);
    if (p.splits < 2) return tail_workspace_bytes(M, N, K);
    return (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float);
}

using BigSquare = BigTile<256, 256, 2, 4, 2>;   // 8 waves of 128 x 64, 2 stages

using BigWide = BigTile<256, 128, 4, 2, 3>;     // 8 waves of 64 x 64, 3 stages
using BigMid = BigTile<128, 128, 2, 2, 2>;      // 4 waves of 64 x 64, 2 stages, 2 per CU

// The split schedule serves the 256 x 256 tile when every M tile is whole and the K-block
// count is even (its two steps per loop turn run unconditionally).
template <class T>
constexpr bool kSplitTile = std::is_same<T, BigSquare>::value;
template <class T>
static bool use_split(int64_t M, int64_t K) {
    return kSplitTile<T> && M % T::BM == 0 && (K / kBlock) % 2 == 0;
}

template <class T>
static void launch_big(const void* a, const float* as, const void* b, const float* bs, void* c,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
    if (use_split<T>(M, K))
        hipLaunchKernelGGL((gemm_big_kernel<T, kSplitTile<T>>), dim3(mt * nt), dim3(T::THREADS), 0, stream,
                           (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, nt);
    else
        hipLaunchKernelGGL((gemm_big_kernel<T, false>), dim3(mt * nt), dim3(T::THREADS), 0, stream,
                           (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, nt);
}

template <class T, int kEpi = kEpiQuant>
static hipError_t launch_quant(const void* a, const float* as, const void* b, const float* bs,
                               void* q, float* qs, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream) {
    const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
    if (kEpi == kEpiQuant && use_split<T>(M, K))
        hipLaunchKernelGGL((gemm_quant_kernel<T, kEpi, kEpi == kEpiQuant && kSplitTile<T>>), dim3(mt * nt),
                           dim3(T::THREADS), 0, stream, (const uint8_t*)a, as, (const uint8_t*)b,
                           bs, (uint8_t*)q, qs, M, N, K, mt, nt);
    else
        hipLaunchKernelGGL((gemm_quant_kernel<T, kEpi, false>), dim3(mt * nt), dim3(T::THREADS),
                           0, stream, (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint8_t*)q,
                           qs, M, N, K, mt, nt);
    return hipGetLastError();
}

// Which kernel configuration serves an M x N x K problem (the tile table).
GemmConfig gemm_config(int64_t M, int64_t N, int64_t /*K*/) {
    const int64_t cus = device_cu_count();
    const int64_t tiles_sq = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t tiles_wide = ((M + 255) / 256) * ((N + 127) / 128);
    // 256 x 256 from 5/8 of a tile per CU up: at 160-288 tiles it beat 256 x 128 by 6-30%
    // (one round of the more efficient tile against several of the smaller one); at 128
    // tiles, half the CUs idle and 256 x 128 is 25% faster.  256 x 128 from one full round
    // of its tiles up; below that, 128 x 128 tiles two per CU were 5-25% faster (2048 x
    // 2048 x 7168: 45.6 against 53.4 us) and even with it at 4096 x 2048 x 7168.
    if (M > 128 && tiles_sq >= cus * 5 / 8) return GemmConfig::kBig256x256;
    if (M > 128 && tiles_wide >= cus) return GemmConfig::kBig256x128;
    return GemmConfig::kBig128x128;
}

const char* gemm_config_name(GemmConfig cfg) {
    switch (cfg) {
        case GemmConfig::kBig256x256: return "lds-direct 256x256, 8 waves of 128x64";
        case GemmConfig::kBig256x128: return "lds-direct 256x128, 8 waves of 64x64";
        case GemmConfig::kBig128x128: return "lds-direct 128x128, 4 waves of 64x64, 2 per CU";
    }
    return "unknown";
}

hipError_t launch_tail_reduce(const float* ws, void* c, int64_t M, int64_t N, int64_t n1,
                              int splits, hipStream_t stream) {
    const int64_t quads = M * (N - n1) / 4;
    int64_t grid = (quads + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    grid = grid < cap ? grid : cap;
    hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ws,
                       (uint16_t*)c, M, N, n1, splits);
    return hipGetLastError();
}

// Whole rounds of 256 x 256 tiles over columns [0, n1), then the tail columns as
// two K halves into the fp32 workspace, then the ordered reduction (tail_plan).
// kHw: the power-of-two-scale GEMM's kernels.
template <bool kHw>
static hipError_t launch_split_last_round(const void* a, const float* as, const void* b,
                                          const float* bs, void* c, int64_t M, int64_t N,
                                          int64_t K, void* workspace, hipStream_t stream) {
    const TailPlan tp = tail_plan(M, N, K);
    const int mt = (int)(M / 256);
    const int64_t n1 = (int64_t)tp.nt_main * 256;
    if constexpr (kHw)
        hipLaunchKernelGGL(gemm_ue8m0_kernel<BigSquare>, dim3(mt * tp.nt_main),
                           dim3(BigSquare::THREADS), 0, stream, (const uint8_t*)a, as,
                           (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, tp.nt_main);
    else if (use_split<BigSquare>(M, K))
        hipLaunchKernelGGL((gemm_big_kernel<BigSquare, true>), dim3(mt * tp.nt_main),
                           dim3(BigSquare::THREADS), 0, stream, (const uint8_t*)a, as,
                           (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, tp.nt_main);
    else
        hipLaunchKernelGGL((gemm_big_kernel<BigSquare, false>), dim3(mt * tp.nt_main),
                           dim3(BigSquare::THREADS), 0, stream, (const uint8_t*)a, as,
                           (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, tp.nt_main);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the split load schedule when both K runs (kb_per blocks and the rest) are even
    if (!kHw && tp.kb_per % 2 == 0 && (K / kBlock - tp.kb_per) % 2 == 0)
        hipLaunchKernelGGL((gemm_tail_kernel<BigSquare, false, true>),
                           dim3(mt * tp.nt_tail * tp.splits), dim3(BigSquare::THREADS), 0, stream,
                           (const uint8_t*)a, as, (const uint8_t*)b, bs, (float*)workspace, M, N,
                           K, mt, tp.nt_tail, n1, tp.kb_per);
    else
        hipLaunchKernelGGL((gemm_tail_kernel<BigSquare, kHw, false>),
                           dim3(mt * tp.nt_tail * tp.splits), dim3(BigSquare::THREADS), 0, stream,
                           (const uint8_t*)a, as, (const uint8_t*)b, bs, (float*)workspace, M, N,
                           K, mt, tp.nt_tail, n1, tp.kb_per);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_tail_reduce((const float*)workspace, c, M, N, n1, tp.splits, stream);
}

hipError_t launch_gemm(const void* a, const float* as, const void* b, const float* bs, void* c,
                       int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    const SplitPlan plan = split_plan(M, N, K);
    if (workspace && plan.splits >= 2 &&
        workspace_bytes >= (size_t)plan.splits * (size_t)M * (size_t)N * sizeof(float)) {
        const int mt = (int)((M + 63) / 64), nt = (int)((N + 63) / 64);
        const size_t lds_bytes = (size_t)plan.kb_per * 2 * 64 * kBlock;
        hipLaunchKernelGGL(gemm_skinny_kernel, dim3(mt * nt, plan.splits), dim3(256), lds_bytes,
                           stream,
                           (const uint8_t*)a, as, (const uint8_t*)b, bs, (float*)workspace, M, N,
                           K, mt, plan.kb_per);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t MN = M * N;
        int64_t grid = (MN + 255) / 256;
        const int64_t cap = (int64_t)device_cu_count() * 8;
        grid = grid < cap ? grid : cap;
        hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                           (const float*)workspace, (uint16_t*)c, MN, plan.splits);
        return hipGetLastError();
    }
    const GemmConfig cfg = gemm_config(M, N, K);
    if (cfg == GemmConfig::kBig256x256 && workspace && tail_plan(M, N, K).splits > 0 &&
        workspace_bytes >= tail_workspace_bytes(M, N, K) && ((uintptr_t)c & 7u) == 0)
        return launch_split_last_round<false>(a, as, b, bs, c, M, N, K, workspace, stream);
    switch (cfg) {
        case GemmConfig::kBig256x256:
            launch_big<BigSquare>(a, as, b, bs, c, M, N, K, stream);
            break;
        case GemmConfig::kBig256x128:
            launch_big<BigWide>(a, as, b, bs, c, M, N, K, stream);
            break;
        case GemmConfig::kBig128x128:
            launch_big<BigMid>(a, as, b, bs, c, M, N, K, stream);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_quant(const void* a, const float* as, const void* b, const float* bs,
                             void* q, float* qs, int64_t M, int64_t N, int64_t K,
                             hipStream_t stream) {
    switch (gemm_config(M, N, K)) {
        case GemmConfig::kBig256x256:
            return launch_quant<BigSquare>(a, as, b, bs, q, qs, M, N, K, stream);
        case GemmConfig::kBig256x128:
            return launch_quant<BigWide>(a, as, b, bs, q, qs, M, N, K, stream);
        case GemmConfig::kBig128x128:
            return launch_quant<BigMid>(a, as, b, bs, q, qs, M, N, K, stream);
    }
    return hipErrorInvalidValue;
}

template <class T>
static hipError_t launch_ue8m0(const void* a, const float* as, const void* b, const float* bs,
                               void* c, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int mt = (int)((M + T::BM - 1) / T::BM), nt = (int)((N + T::BN - 1) / T::BN);
    hipLaunchKernelGGL(gemm_ue8m0_kernel<T>, dim3(mt * nt), dim3(T::THREADS), 0, stream,
                       (const uint8_t*)a, as, (const uint8_t*)b, bs, (uint16_t*)c, M, N, K, mt, nt);
    return hipGetLastError();
}

// The power-of-two-scale GEMM takes a workspace only for the split last round.
size_t gemm_ue8m0_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    return tail_workspace_bytes(M, N, K);
}

hipError_t launch_gemm_ue8m0(const void* a, const float* as, const void* b, const float* bs,
                             void* c, int64_t M, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    const GemmConfig cfg = gemm_config(M, N, K);
    if (cfg == GemmConfig::kBig256x256 && workspace && tail_plan(M, N, K).splits > 0 &&
        workspace_bytes >= tail_workspace_bytes(M, N, K) && ((uintptr_t)c & 7u) == 0)
        return launch_split_last_round<true>(a, as, b, bs, c, M, N, K, workspace, stream);
    switch (cfg) {
        case GemmConfig::kBig256x256: return launch_ue8m0<BigSquare>(a, as, b, bs, c, M, N, K, stream);
        // the e8m0 loop has no fold: 128 x 128 tiles two per CU measured 6% faster than
        // 256 x 128 here too (4096 x 2048 x 7168)
        case GemmConfig::kBig256x128: return launch_ue8m0<BigMid>(a, as, b, bs, c, M, N, K, stream);
        case GemmConfig::kBig128x128: return launch_ue8m0<BigMid>(a, as, b, bs, c, M, N, K, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_swiglu_quant(const void* a, const float* as, const void* w13,
                                    const float* s13, void* q, float* qs, int64_t M, int64_t n_out,
                                    int64_t K, hipStream_t stream) {
    return launch_quant<BigSquare, kEpiSwiglu>(a, as, w13, s13, q, qs, M, 2 * n_out, K, stream);
}

// The no-allocation GEMM: the workspace bfp8_gemm takes from its caller (the
// split-K partial sums of skinny problems and the split last round of large
// ones) lives instead in this fixed device array, one per GPU, held until the
// process ends.  64 MiB covers every shape whose last round is split (at most
// 2 x 128 tiles of 256 x 256 fp32 partials) and the skinny split plans up to
// that size.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in): its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and that
// address is what the kernels receive.  Every call on one GPU shares the
// array, so calls that overlap on one GPU (different streams, no ordering)
// race on it.  No kernel needs it zeroed: every partial is written before it
// is read.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_gemm_noalloc(const void* a, const float* as, const void* b, const float* bs,
                               void* c, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const size_t need = gemm_workspace_bytes(M, N, K);
    if (need > kNoAllocScratchBytes) return hipErrorInvalidValue;   // rejected by the ABI first
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) return e;
    }
    // the same plans and kernels as launch_gemm with a caller workspace of `need` bytes
    return launch_gemm(a, as, b, bs, c, M, N, K, ws, need, stream);
}

}  // namespace bfp8
