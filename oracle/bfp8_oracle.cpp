/*
 * bfp8_oracle.cpp - plain, slow CPU oracle for the block-scaled FP8 linear path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or constant with
 * the HIP library.
 *
 * What it computes, and where the pages state it:
 *   - "Data flow - deepseek-ai/DeepSeek-V3" (codevetter), the FP8
 *     quantization bullet: act_quant yields a float8_e4m3fn tensor plus fp32
 *     scales, one per 128-element block; fp8_gemm multiplies the scaled
 *     blocks and accumulates in fp32; each 1-byte Linear weight carries a
 *     .scale tensor.
 *   - pyshine "DeepSeek-V3" tour, "The Three Ideas That Make V3 Fast",
 *     paragraph "FP8 with per-block scales": weights are e4m3 with a grid of
 *     per-128-block scales; act_quant clamps each tile's max and divides it
 *     by 448 (the e4m3 ceiling); weight_dequant expands weights for an
 *     ordinary BF16 matmul; fp8_gemm accumulates FP8 products rescaled by
 *     their block scales.
 *   - "Behavior traces" (codevetter), the fp8->bf16 trace bullet: each
 *     1-byte tensor is dequantized with its (renamed) scale_inv, i.e. the
 *     stored scale is a multiplier.
 *   - "Behavior traces" (codevetter), the MoE trace bullet: per-expert token
 *     counts; for each local expert with tokens, the tokens routed to it are
 *     selected in ascending order, run through the expert, and added into a
 *     zero-initialised y after multiplication by their routing weight.
 *     "Data flow" (codevetter): a GPU holds a contiguous range of experts.
 *   - pyshine tour, "FP8 with per-block scales": the second branch of
 *     linear() dequantizes the weight and runs an ordinary BF16 matmul.
 *   - the gated FFN (w1, w3 -> activation * up -> w2) of the MLP/Expert
 *     modules ("Data flow", MLP and Expert projections); the activation is
 *     this oracle's stated reading (SiLU), the pages do not print it.
 * The e4m3 format itself is the OCP 8-bit floating point E4M3 encoding
 * (torch.float8_e4m3fn): bias 7, no infinities, NaN only at S.1111.111,
 * largest finite value 448.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): the clamp is a lower floor ORACLE_AMAX_FLOOR on the block
 * max; the quantizer divides in IEEE fp32 and then rounds to nearest-even
 * with saturation at +-448; weight scales tile the weight in 128x128 blocks;
 * the GEMM reference is accumulated in fp64; the MoE combine sums in fp64
 * (the pages accumulate y in the activation dtype, expert by expert).
 *
 * Parity status: every function here is pinned by the CPU tests against
 * brute force, closed forms, torch's own e4m3/bf16 casts or exact rational
 * arithmetic, except the value of ORACLE_AMAX_FLOOR (the pages give none),
 * which is "parity unpinned".
 *
 * Plain C++17: loops over rows and elements, std::thread over output rows for
 * the GEMM references, every export extern "C" so ctypes can load it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <thread>
#include <vector>

#define ORACLE_BLOCK 128
#define ORACLE_E4M3_MAX 448.0f
#define ORACLE_AMAX_FLOOR 1e-4f

/* Runs worker(jobs[t]) for t = 0 .. n-1, job 0 on the calling thread; a job
 * whose thread cannot be started runs on the calling thread too. */
template <class Job, class Fn>
static void run_jobs(std::vector<Job>& jobs, Fn worker) {
    std::vector<std::thread> th;
    size_t t = 1;
    try {
        for (; t < jobs.size(); ++t) th.emplace_back(worker, &jobs[t]);
    } catch (...) {
        for (; t < jobs.size(); ++t) worker(&jobs[t]);
    }
    worker(&jobs[0]);
    for (auto& x : th) x.join();
}

extern "C" {

/* ---------------------------------------------------------------- formats */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the upper half of a binary32, so widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
 * Written as: keep the upper 16 bits, and add one unit in the last kept place
 * when the dropped half is above one half, or exactly one half and the kept
 * part is odd. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u = f32_to_bits(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* e4m3 code -> value.  Layout s.eeee.mmm, bias 7:
 *   E == 0          : subnormal  m * 2^-9
 *   E in 1..15      : (1 + m/8) * 2^(E-7)
 *   E == 15, m == 7 : NaN (no infinities) */
float oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7, E = (c >> 3) & 15, m = c & 7;
    float mag;
    if (E == 15 && m == 7) return sign ? -NAN : NAN;
    if (E == 0) mag = ldexpf((float)m, -9);
    else mag = ldexpf(1.0f + (float)m / 8.0f, E - 7);
    return sign ? -mag : mag;
}

/* value -> e4m3 code, round to nearest with ties to even, saturating at the
 * largest finite magnitude 448 (code 0x7E).  The sign is kept, so a negative
 * value that rounds to zero gives 0x80. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;               /* outside the contract */
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;             /* saturate (also +-inf) */
    if (a == 0.0) return sign;
    /* binade of a, limited below by the smallest normal exponent -6 */
    int e2;
    frexp(a, &e2);                                  /* a = f * 2^e2, f in [0.5,1) */
    int E = e2 - 1;                                 /* floor(log2 a) */
    if (E < -6) E = -6;
    double quantum = ldexp(1.0, E - 3);             /* spacing of 3-bit mantissas */
    double r = a / quantum;                         /* exact: power-of-two scaling */
    double n = floor(r);
    double frac = r - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    double mag = n * quantum;                       /* nearest representable */
    if (mag == 0.0) return sign;
    if (mag < ldexp(1.0, -6))                       /* subnormal: m * 2^-9 */
        return sign | (uint8_t)(mag / ldexp(1.0, -9));
    int e3;
    frexp(mag, &e3);
    int Eb = e3 - 1;                                /* may have carried upward */
    double mant = mag / ldexp(1.0, Eb);             /* in [1, 2) */
    int m = (int)((mant - 1.0) * 8.0);
    return sign | (uint8_t)(((Eb + 7) << 3) | m);
}

void oracle_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(const uint8_t* c, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

void oracle_f32_to_bf16_array(const float* v, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(v[i]);
}

float oracle_amax_floor(void) { return ORACLE_AMAX_FLOOR; }

/* ------------------------------------------------------------- act_quant */

/* For each row m and each 128-wide block kb of the last dimension:
 *   amax = max |x| over the block (exact, on the bf16 values)
 *   s    = max(amax, ORACLE_AMAX_FLOOR) / 448        (fp32 division)
 *   q    = e4m3(x / s)                               (fp32 division, then RNE+sat)
 * x is bf16 [M,K] row-major, q is [M,K], s is [M, K/128].
 * Returns 0, or -1 when K is not a multiple of 128. */
int oracle_act_quant(const uint16_t* x, uint8_t* q, float* s, int64_t M, int64_t K) {
    if (K <= 0 || K % ORACLE_BLOCK != 0 || M < 0) return -1;
    int64_t KB = K / ORACLE_BLOCK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint16_t* xb = x + m * K + kb * ORACLE_BLOCK;
            uint8_t* qb = q + m * K + kb * ORACLE_BLOCK;
            float amax = 0.0f;
            for (int j = 0; j < ORACLE_BLOCK; ++j) {
                float a = fabsf(oracle_bf16_to_f32(xb[j]));
                if (a > amax) amax = a;
            }
            float clamped = amax < ORACLE_AMAX_FLOOR ? ORACLE_AMAX_FLOOR : amax;
            float scale = clamped / ORACLE_E4M3_MAX;
            for (int j = 0; j < ORACLE_BLOCK; ++j) {
                float quotient = oracle_bf16_to_f32(xb[j]) / scale;
                qb[j] = oracle_e4m3_encode(quotient);
            }
            s[m * KB + kb] = scale;
        }
    }
    return 0;
}

/* act_quant with power-of-two scales: the reading of the model's scale_fmt
 * field ("Data flow", config data flows: scale_fmt is a ModelArgs field; its
 * meaning is not on the pages).  Reading: the block scale max(amax, floor)/448
 * (an fp32 division, as above) is rounded UP to the next power of two, so
 * every quotient still fits the e4m3 range; the scale is then exactly
 * representable as an unsigned 8-bit exponent (e8m0).  The power is found
 * with frexp: y = f 2^e with f in [0.5, 1), so 2^e is the smallest power of
 * two >= y unless f == 0.5 (y itself a power of two). */
int oracle_act_quant_pow2(const uint16_t* x, uint8_t* q, float* s, int64_t M, int64_t K) {
    if (K <= 0 || K % ORACLE_BLOCK != 0 || M < 0) return -1;
    int64_t KB = K / ORACLE_BLOCK;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint16_t* xb = x + m * K + kb * ORACLE_BLOCK;
            uint8_t* qb = q + m * K + kb * ORACLE_BLOCK;
            float amax = 0.0f;
            for (int j = 0; j < ORACLE_BLOCK; ++j) {
                float a = fabsf(oracle_bf16_to_f32(xb[j]));
                if (a > amax) amax = a;
            }
            float clamped = amax < ORACLE_AMAX_FLOOR ? ORACLE_AMAX_FLOOR : amax;
            float y = clamped / ORACLE_E4M3_MAX;
            int e;
            double f = frexp((double)y, &e);
            float scale = (float)ldexp(1.0, f == 0.5 ? e - 1 : e);
            for (int j = 0; j < ORACLE_BLOCK; ++j) {
                float quotient = oracle_bf16_to_f32(xb[j]) / scale;
                qb[j] = oracle_e4m3_encode(quotient);
            }
            s[m * KB + kb] = scale;
        }
    }
    return 0;
}

/* -------------------------------------------------------- weight_dequant */

/* out[n,k] = bf16( e4m3_value(w[n,k]) * S[n/128][k/128] ), the product
 * rounded once to fp32 and then once to bf16.  w is [N,K], S is
 * [ceil(N/128), ceil(K/128)], out is bf16 [N,K]. */
void oracle_weight_dequant(const uint8_t* w, const float* S, uint16_t* out,
                           int64_t N, int64_t K) {
    int64_t KB = (K + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float scale = S[(n / ORACLE_BLOCK) * KB + k / ORACLE_BLOCK];
            float product = oracle_e4m3_decode(w[n * K + k]) * scale;
            out[n * K + k] = oracle_f32_to_bf16(product);
        }
}

/* ------------------------------------------------------------------ GEMM */

/* ref[m,n] = sum over blocks kb of
 *              ( sum_{k in kb} a[m,k] * b[n,k] ) * sa[m,kb] * sb[n/128,kb]
 * in fp64.  a is e4m3 [M,K], sa is [M,K/128], b is e4m3 [N,K] (a Linear
 * weight, out_features x in_features, so C = A * B^T), sb is
 * [ceil(N/128), K/128].  The per-block sum of e4m3 products is exact in fp64
 * (each product is an integer multiple of 2^-18 below 2^18 in size, and 128 of
 * them stay below 2^53 units).  Only the listed rows are computed, into
 * out[i*N + n] for rows[i]. */
struct gemm_job {
    const uint8_t *a, *b;
    const float *sa, *sb;
    int64_t N, K;
    const int32_t* off;   /* grouped only: int32 [G+1] row offsets, else NULL */
    int32_t G;
    const int64_t* rows;
    int64_t nrows;
    double* out;
    int tid, nthreads;
    float table[256];
};

static void gemm_row(const gemm_job* J, const uint8_t* b, const float* sb,
                     int64_t m, double* out_row) {
    int64_t KB = J->K / ORACLE_BLOCK;
    const uint8_t* arow = J->a + m * J->K;
    for (int64_t n = 0; n < J->N; ++n) {
        const uint8_t* brow = b + n * J->K;
        double total = 0.0;
        for (int64_t kb = 0; kb < KB; ++kb) {
            double block_sum = 0.0;
            for (int j = 0; j < ORACLE_BLOCK; ++j) {
                int64_t k = kb * ORACLE_BLOCK + j;
                block_sum += (double)J->table[arow[k]] * (double)J->table[brow[k]];
            }
            total += block_sum * (double)J->sa[m * KB + kb]
                               * (double)sb[(n / ORACLE_BLOCK) * KB + kb];
        }
        out_row[n] = total;
    }
}

static void gemm_worker(gemm_job* J) {
    int64_t KB = J->K / ORACLE_BLOCK;
    int64_t NB = (J->N + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
    for (int64_t i = J->tid; i < J->nrows; i += J->nthreads) {
        int64_t m = J->rows[i];
        double* out_row = J->out + i * J->N;
        if (!J->off) { gemm_row(J, J->b, J->sb, m, out_row); continue; }
        int32_t g = -1;
        for (int32_t h = 0; h < J->G; ++h)
            if (m >= J->off[h] && m < J->off[h + 1]) { g = h; break; }
        if (g < 0) {
            for (int64_t n = 0; n < J->N; ++n) out_row[n] = NAN;
            continue;
        }
        gemm_row(J, J->b + (int64_t)g * J->N * J->K, J->sb + (int64_t)g * NB * KB,
                 m, out_row);
    }
}

static int run_gemm_rows(const uint8_t* a, const float* sa, const uint8_t* b,
                         const float* sb, const int32_t* off, int32_t G,
                         int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                         double* out, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    std::vector<gemm_job> jobs((size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        gemm_job* J = &jobs[t];
        J->a = a; J->b = b; J->sa = sa; J->sb = sb; J->N = N; J->K = K;
        J->off = off; J->G = G;
        J->rows = rows; J->nrows = nrows; J->out = out;
        J->tid = t; J->nthreads = nthreads;
        for (int c = 0; c < 256; ++c) J->table[c] = oracle_e4m3_decode((uint8_t)c);
    }
    run_jobs(jobs, gemm_worker);
    return 0;
}

int oracle_gemm_rows(const uint8_t* a, const float* sa, const uint8_t* b,
                     const float* sb, int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    if (K <= 0 || K % ORACLE_BLOCK != 0 || M < 0 || N < 0) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return -1;
    return run_gemm_rows(a, sa, b, sb, NULL, 0, N, K, rows, nrows, out, nthreads);
}

/* Grouped GEMM: rows [off[g], off[g+1]) of a (and sa) are multiplied by
 * expert g's weight b[g] with its scale grid sb[g].  For each requested row
 * the owning group is found from the offsets; a row that lies in no group
 * yields NaN in every column.  b is [G,N,K], sb is [G, ceil(N/128), K/128],
 * off is int32 [G+1]. */
int oracle_gemm_grouped_rows(const uint8_t* a, const float* sa, const uint8_t* b,
                             const float* sb, const int32_t* off, int32_t G,
                             int64_t total_M, int64_t N, int64_t K,
                             const int64_t* rows, int64_t nrows, double* out,
                             int nthreads) {
    if (K <= 0 || K % ORACLE_BLOCK != 0 || G < 1 || N < 0 || total_M < 0) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= total_M) return -1;
    return run_gemm_rows(a, sa, b, sb, off, G, N, K, rows, nrows, out, nthreads);
}

/* --------------------------------------------------------- BF16 branch GEMM */

/* The other branch of linear(): the weight is first expanded to bf16
 * (weight_dequant) and multiplied with the bf16 activations by an ordinary
 * BF16 matmul (pyshine tour, "FP8 with per-block scales").  Reference:
 *     out[i, n] = sum_k a[rows[i], k] * b[n, k]   in fp64,
 * a bf16 [M,K], b bf16 [N,K] (bit patterns), C = A * B^T.  Each product of
 * two bf16 values is exact in fp64; only the sum rounds. */
struct gemm_bf16_job {
    const uint16_t *a, *b;
    int64_t N, K;
    const int64_t* rows;
    int64_t nrows;
    double* out;
    int tid, nthreads;
};

static void gemm_bf16_worker(gemm_bf16_job* J) {
    std::vector<double> arow((size_t)J->K);
    for (int64_t i = J->tid; i < J->nrows; i += J->nthreads) {
        const uint16_t* a = J->a + J->rows[i] * J->K;
        for (int64_t k = 0; k < J->K; ++k) arow[k] = (double)oracle_bf16_to_f32(a[k]);
        for (int64_t n = 0; n < J->N; ++n) {
            const uint16_t* b = J->b + n * J->K;
            double sum = 0.0;
            for (int64_t k = 0; k < J->K; ++k) sum += arow[k] * (double)oracle_bf16_to_f32(b[k]);
            J->out[i * J->N + n] = sum;
        }
    }
}

int oracle_gemm_bf16_rows(const uint16_t* a, const uint16_t* b, int64_t M, int64_t N, int64_t K,
                          const int64_t* rows, int64_t nrows, double* out, int nthreads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    std::vector<gemm_bf16_job> jobs((size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        gemm_bf16_job* J = &jobs[t];
        J->a = a; J->b = b; J->N = N; J->K = K;
        J->rows = rows; J->nrows = nrows; J->out = out;
        J->tid = t; J->nthreads = nthreads;
    }
    run_jobs(jobs, gemm_bf16_worker);
    return 0;
}

/* ------------------------------------------------------- gated FFN activation */

/* The gated FFN between the first and the second projection of an expert
 * or the dense MLP: h = silu(w1 x) * (w3 x).  The pages name w1/w2/w3
 * ("gate_proj -> w1") but never print the activation; this oracle takes
 * SiLU, silu(x) = x / (1 + e^-x), as DeepSeek-V3's model code uses.  The
 * steps follow a bf16 model: g and u are the projections' bf16 outputs,
 * silu(g) is evaluated in floating point and rounded to bf16, and the product
 * of the two bf16 values (exact) is rounded to bf16:
 *     h = bf16( bf16( silu( bf16(g) ) ) * bf16(u) ).
 * g and u arrive as fp64 GEMM results and are rounded to bf16 through fp32.
 * Output: bf16 bit patterns. */
void oracle_swiglu_bf16(const double* g, const double* u, int64_t n, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) {
        const double gb = (double)oracle_bf16_to_f32(oracle_f32_to_bf16((float)g[i]));
        const double ub = (double)oracle_bf16_to_f32(oracle_f32_to_bf16((float)u[i]));
        const double sg = gb / (1.0 + exp(-gb));
        const double sgb = (double)oracle_bf16_to_f32(oracle_f32_to_bf16((float)sg));
        h[i] = oracle_f32_to_bf16((float)(sgb * ub));
    }
}

/* ------------------------------------------------- MoE dispatch and combine */

/* Dispatch of one GPU's share of routed experts ("Behavior traces", MoE
 * trace: for each local expert with tokens, the tokens routed to it, in
 * ascending order, are gathered; "Data flow", Expert sharding: the local
 * experts are a contiguous range of expert ids).
 *   topk: int32 [T, topk] expert ids per token; local experts are
 *         expert_lo .. expert_lo + G - 1.
 * Outputs: offsets [G+1] (rows of local expert g are offsets[g] ..
 * offsets[g+1]); row_token [offsets[G]] (token of each gathered row);
 * slot_row [T, topk] (gathered row of each (token, slot), -1 when the slot's
 * expert is not local).  Written as the pages' loop: expert by expert, token
 * by token. */
void oracle_moe_dispatch(const int32_t* topk, int64_t T, int32_t k, int32_t expert_lo,
                         int32_t G, int32_t* offsets, int32_t* row_token, int32_t* slot_row) {
    for (int64_t i = 0; i < T * k; ++i) slot_row[i] = -1;
    int32_t row = 0;
    for (int32_t g = 0; g < G; ++g) {
        offsets[g] = row;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t j = 0; j < k; ++j)
                if (topk[t * k + j] == expert_lo + g) {
                    row_token[row] = (int32_t)t;
                    slot_row[t * k + j] = row;
                    ++row;
                }
    }
    offsets[G] = row;
}

/* Combine: y[t, n] = sum over slots j with slot_row[t, j] >= 0 of
 *          weight[t, j] * out[slot_row[t, j], n], in fp64.
 * out is bf16 [rows, N] (the grouped GEMM's output), y is fp64 [T, N]. */
void oracle_moe_combine(const uint16_t* out, const int32_t* slot_row, const float* weight,
                        int64_t T, int32_t k, int64_t N, double* y) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                const int32_t r = slot_row[t * k + j];
                if (r >= 0)
                    acc += (double)weight[t * k + j] * (double)oracle_bf16_to_f32(out[(int64_t)r * N + n]);
            }
            y[t * N + n] = acc;
        }
}

}  /* extern "C" */
