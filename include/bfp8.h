/*
 * bfp8.h - C ABI of the block-scaled FP8 linear path on AMD Instinct MI355X (gfx950).
 *
 * The path is the FP8 branch of DeepSeek-V3's quantization-aware linear():
 * activations are quantized to e4m3 with one fp32 scale per 128-element block
 * (act_quant), weights are e4m3 with one fp32 scale per 128x128 block, the
 * GEMM multiplies the scaled blocks and accumulates in fp32 (fp8_gemm), and
 * weights can be expanded to bf16 for an ordinary BF16 matmul
 * (weight_dequant).  Sources:
 *   [DF]  "Data flow - deepseek-ai/DeepSeek-V3" (codevetter), bullet
 *         "FP8 quantization data flow".
 *   [BT]  "Behavior traces - deepseek-ai/DeepSeek-V3" (codevetter), bullets
 *         "MoE trace" and "fp8->bf16 trace".
 *   [PY]  pyshine "DeepSeek-V3" tour, section "The Three Ideas That Make V3
 *         Fast", paragraph "FP8 with per-block scales", and section "Honest
 *         Limits" (Python expert loop vs a fused grouped GEMM).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer to row-major, densely packed
 *     memory owned by the caller.  The library never allocates, frees or
 *     keeps a pointer after the call returns.  The one exception is the fixed
 *     device array behind bfp8_gemm_noalloc (see there).
 *   - e4m3 means the OCP FP8 E4M3 format (torch.float8_e4m3fn): bias 7, no
 *     infinities, largest finite value 448 (code 0x7E); one byte per element.
 *   - bf16 is the upper half of an IEEE binary32; two bytes per element.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is only enqueued; no call synchronizes.  Faults inside a kernel
 *     surface at the caller's next synchronization, as with any HIP launch.
 *   - Arguments are validated on the host BEFORE any HIP call; a rejected call
 *     launches nothing and returns the status code.  A zero-sized problem
 *     (M == 0, N == 0, total_M == 0) returns BFP8_OK without a launch.
 *   - Outputs must not alias inputs.  Calls on different streams that write
 *     different outputs may overlap; the library keeps no state between calls
 *     (bfp8_gemm_noalloc's scratch array aside).
 *   - Block edge: BFP8_BLOCK = 128 everywhere (every call site on the pages uses
 *     128-element activation blocks and a 128x128 weight-scale grid).
 */
#ifndef BFP8_H
#define BFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BFP8_BLOCK 128
#define BFP8_VERSION 8
/* bytes of the device scratch array behind bfp8_gemm_noalloc (per GPU) */
#define BFP8_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
#define BFP8_MOE_MAX_GROUPS 1024

typedef enum bfp8_status {
    BFP8_OK = 0,
    BFP8_ERR_NULL = 1,      /* a required pointer is NULL */
    BFP8_ERR_SHAPE = 2,     /* a size is negative, K is not a multiple of 128 where required,
                               or a size is past the limit its call states */
    BFP8_ERR_ALIGN = 3,     /* a pointer is not aligned as documented */
    BFP8_ERR_WORKSPACE = 4, /* workspace smaller than the matching *_workspace_size() */
    BFP8_ERR_GROUPS = 5,    /* G < 1, or G > BFP8_MOE_MAX_GROUPS (MoE dispatch) */
    BFP8_ERR_HIP = 6,       /* the HIP runtime reported an error at launch */
    BFP8_ERR_ARG = 7,       /* any other invalid argument */
    BFP8_ERR_SCRATCH = 8    /* bfp8_gemm_noalloc: the problem needs more than
                               BFP8_NOALLOC_SCRATCH_BYTES of scratch */
} bfp8_status;

/* act_quant ([DF] FP8 bullet; [PY] "FP8 with per-block scales").
 * For each row m and each 128-element block kb of the last dimension:
 *     amax  = max |x[m, 128kb + j]|                       (exact, on bf16 values)
 *     s     = max(amax, 1e-4f) / 448                      (fp32, correctly rounded)
 *     q[..] = e4m3_rne_saturating( x[..] / s )            (fp32 quotient, correctly rounded)
 *     scales[m, kb] = s
 * The floor 1e-4 on amax is this library's reading of "clamping each tile's
 * max" (it only matters for blocks whose max |x| is below 1e-4).  Inputs are
 * finite: a block holding a NaN or an infinity gets unspecified codes and
 * scale (the call itself still succeeds and writes only its outputs).
 *   x_bf16 : bf16 [M, K], 16-byte aligned
 *   q_e4m3 : e4m3 [M, K] output, 16-byte aligned
 *   scales : fp32 [M, K/128] output, 4-byte aligned
 * Errors: BFP8_ERR_SHAPE if M < 0, K <= 0 or K % 128 != 0; BFP8_ERR_NULL if a
 * pointer is NULL while M > 0; BFP8_ERR_ALIGN on misalignment. */
int bfp8_act_quant(const void* x_bf16, void* q_e4m3, float* scales,
                   int64_t M, int64_t K, void* stream);

/* weight_dequant ([PY] "FP8 with per-block scales": dequantize then an
 * ordinary BF16 matmul; [BT] "fp8->bf16 trace": each 1-byte tensor is
 * dequantized with its scale, which is a multiplier).
 *     out[n, k] = bf16_rne( fp32( e4m3_value(w[n, k]) * s[n/128, k/128] ) )
 *   w_e4m3  : e4m3 [N, K]
 *   s       : fp32 [ceil(N/128), ceil(K/128)]; partial edge blocks allowed
 *   out_bf16: bf16 [N, K] output
 * Any N, K >= 0.  A vectorized kernel is used when K % 8 == 0, N*K is a
 * multiple of 1024, w is 8-byte and out 16-byte aligned; a scalar one otherwise.
 * Errors: BFP8_ERR_SHAPE if N < 0 or K < 0; BFP8_ERR_NULL for a NULL pointer
 * when N*K > 0; BFP8_ERR_ALIGN if out is not 2-byte or s not 4-byte aligned. */
int bfp8_weight_dequant(const void* w_e4m3, const float* s, void* out_bf16,
                        int64_t N, int64_t K, void* stream);

/* fp8_gemm ([DF] "fp8_gemm multiplies scaled blocks accumulating in fp32";
 * [PY] products of FP8 operands rescaled by their block scales).
 * C = A * B^T with B a Linear weight (out_features x in_features):
 *     c[m, n] = bf16_rne( sum_kb ( sum_{k in kb} a[m,k] * b[n,k] ) * a_s[m,kb] * b_s[n/128,kb] )
 * where each inner 128-term block product runs on fp8 MFMA into a fresh fp32
 * accumulator and is folded into the running fp32 sum with its two scales.
 *   a   : e4m3 [M, K], 16-byte aligned         a_s : fp32 [M, K/128]
 *   b   : e4m3 [N, K], 16-byte aligned         b_s : fp32 [ceil(N/128), K/128]
 *   c_bf16 : bf16 [M, N] output, 4-byte aligned (N odd: 2-byte)
 *   workspace : optional fp32 scratch: split-K partial sums on skinny problems
 *     (M <= 64, or M <= 256 with at most 32 output tiles of 128 x 128), and on
 *     large problems (K >= 80 * 128) whose last round of 256 x 256 tiles is at
 *     most half full, the partial sums of those tiles' two K halves.  NULL
 *     disables both (one pass over K per tile).  If non-NULL it must hold at
 *     least bfp8_gemm_workspace_size(M, N, K) bytes and be 16-byte aligned;
 *     its contents on entry do not matter.
 * Errors: BFP8_ERR_SHAPE if M, N < 0, K <= 0, K % 128 != 0 or K >= 2^22 (the
 * tiles address rows with 32-bit byte offsets); BFP8_ERR_NULL; BFP8_ERR_ALIGN;
 * BFP8_ERR_WORKSPACE if workspace_bytes is too small. */
int bfp8_gemm(const void* a, const float* a_s, const void* b, const float* b_s,
              void* c_bf16, int64_t M, int64_t N, int64_t K,
              void* workspace, size_t workspace_bytes, void* stream);

/* bfp8_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels and results (bit for bit) as bfp8_gemm with a workspace
 * of bfp8_gemm_workspace_size(M, N, K) bytes, but that workspace is a
 * library-owned device array of BFP8_NOALLOC_SCRATCH_BYTES (64 MiB), one per
 * GPU, reserved when the library's code is loaded on that GPU and held until
 * the process ends.  The call itself allocates nothing (no hipMalloc, hipFree
 * or allocating library routine); its first call on a device looks up that
 * device's array address, with that device current.  `stream` must belong to
 * the current device.  Every call on one GPU shares its array and leaves its
 * contents behind: calls that may overlap on one GPU (different streams with
 * no ordering between them) race on it and must not be issued.  Nothing in the
 * array needs to start at zero.
 * Errors: as bfp8_gemm, plus BFP8_ERR_SCRATCH if bfp8_gemm_workspace_size(M,
 * N, K) exceeds BFP8_NOALLOC_SCRATCH_BYTES (checked before any HIP call; the
 * problem can still run through bfp8_gemm with a caller workspace, or with
 * none). */
int bfp8_gemm_noalloc(const void* a, const float* a_s, const void* b, const float* b_s,
                      void* c_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* fp8_gemm with the next linear()'s act_quant fused into its epilogue ([DF]
 * FP8 bullet: a linear() output is quantized in 128-element blocks before the
 * next fp8_gemm; the dense chain's "act_quant of W1 output before the second
 * GEMM").  Same product as bfp8_gemm, but instead of bf16 C it writes
 *     q, qs = act_quant( bf16_rne(C) )
 * i.e. exactly what bfp8_act_quant would write for bfp8_gemm's output, bit for
 * bit, without storing or re-reading C.
 *   a, a_s, b, b_s : as bfp8_gemm
 *   q_e4m3  : e4m3 [M, N] output, 4-byte aligned
 *   q_scales: fp32 [M, N/128] output
 * Errors: as bfp8_gemm, and BFP8_ERR_SHAPE if N % 128 != 0. */
int bfp8_gemm_act_quant(const void* a, const float* a_s, const void* b, const float* b_s,
                        void* q_e4m3, float* q_scales, int64_t M, int64_t N, int64_t K,
                        void* stream);

/* The gated FFN's first projection with its activation and act_quant fused
 * into the epilogue (the MLP/Expert modules' w1 and w3 ([DF]), then the next
 * linear()'s act_quant).  The pages do not print the activation; this
 * library reads it as SiLU, silu(x) = x / (1 + e^-x), with the rounding steps
 * of a bf16 model:
 *     g = bf16(x w1^T),  u = bf16(x w3^T)          (block-scaled fp8 GEMMs)
 *     h = bf16( bf16( silu(g) ) * u )              (silu in fp32)
 *     q, q_scales = act_quant(h)                   (128-element blocks)
 * The weight is w1 and w3 interleaved by 64 rows: rows 128 t .. 128 t + 63
 * of w13 are w1 rows 64 t .., rows 128 t + 64 .. 128 t + 127 are w3 rows
 * 64 t .. (bfp8.interleave_w13 builds it once from w1, w3 and their scale
 * grids).  Its scales are one per 64 weight rows: s13[2 t + 0, kb] =
 * w1_s[t / 2, kb], s13[2 t + 1, kb] = w3_s[t / 2, kb].
 *   a, a_s   : as bfp8_gemm (x quantized by act_quant)
 *   w13      : e4m3 [2 N, K], 16-byte aligned     s13 : fp32 [2 N / 64, K/128]
 *   q_e4m3   : e4m3 [M, N] output, 4-byte aligned q_scales : fp32 [M, N/128]
 * Errors: as bfp8_gemm, and BFP8_ERR_SHAPE if N % 128 != 0. */
int bfp8_gemm_swiglu_act_quant(const void* a, const float* a_s, const void* w13,
                               const float* s13, void* q_e4m3, float* q_scales, int64_t M,
                               int64_t N, int64_t K, void* stream);

/* Power-of-two scales: the library's reading of the model's scale_fmt field
 * ([DF] config data flows: scale_fmt is a ModelArgs field; the pages do not
 * say what it means).  Reading: each block scale is rounded UP to a power of
 * two (an unsigned 8-bit exponent, "ue8m0"), so every quotient stays in the
 * e4m3 range and the scales can be applied by the hardware.
 *
 * bfp8_act_quant_ue8m0: as bfp8_act_quant, but
 *     s = 2^ceil(log2( max(amax, 1e-4f) / 448 ))   (the fp32 quotient rounded up
 *                                                   to a power of two, exactly)
 * Same arguments, layouts and errors as bfp8_act_quant. */
int bfp8_act_quant_ue8m0(const void* x_bf16, void* q_e4m3, float* scales, int64_t M, int64_t K,
                         void* stream);

/* bfp8_gemm_ue8m0: fp8_gemm for power-of-two activation and weight scales.
 * The MFMA applies the scales (its e8m0 scale operands) and accumulates the
 * scaled block products directly, with no per-block fold:
 *     c[m, n] = bf16_rne( sum_kb P_kb[m, n] * a_s[m, kb] * b_s[n/128, kb] )
 * Every scale must be a power of two in [2^-127, 2^127] stored as fp32 (as
 * bfp8_act_quant_ue8m0 writes); for any other value only its exponent is used.
 * Same arguments, layouts and errors as bfp8_gemm, except that the optional
 * workspace serves only large problems (K >= 80 * 128) whose last round of
 * 256 x 256 tiles is at most half full (the partial sums of those tiles' two
 * K halves); it must hold bfp8_gemm_ue8m0_workspace_size(M, N, K) bytes
 * (BFP8_ERR_WORKSPACE otherwise), 16-byte aligned, contents irrelevant. */
int bfp8_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s,
                    void* c_bf16, int64_t M, int64_t N, int64_t K, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Bytes of fp32 workspace bfp8_gemm_ue8m0 would use at this shape (0 when its
 * last round is not split).  Pure host function (planned for the 256 CUs of
 * MI355X). */
size_t bfp8_gemm_ue8m0_workspace_size(int64_t M, int64_t N, int64_t K);

/* The FP8 branch of linear() in one call ([DF] FP8 bullet: act_quant of the
 * input, then fp8_gemm with the weight and its scale):
 *     y = bf16( fp8_gemm( act_quant(x), w, w_s ) )
 * It runs bfp8_act_quant into the workspace, then bfp8_gemm with the rest of
 * the workspace as its split-K partials, so y is bit-identical to those two
 * calls (with a split-K workspace where bfp8_gemm would split).
 *   x_bf16 : bf16 [M, K], 16-byte aligned;  w, w_s : as bfp8_gemm's b, b_s
 *   y_bf16 : bf16 [M, N] output
 *   workspace : DEVICE, at least bfp8_linear_fp8_workspace_size(M, N, K)
 *     bytes, 256-byte aligned, owned by the caller, any contents; it holds the
 *     codes, the scales and the split partials of the call.  Calls that share
 *     a workspace must not overlap in time.
 * Errors: as bfp8_gemm; BFP8_ERR_NULL if the workspace is NULL;
 * BFP8_ERR_WORKSPACE if it is too small. */
size_t bfp8_linear_fp8_workspace_size(int64_t M, int64_t N, int64_t K);
int bfp8_linear_fp8(const void* x_bf16, const void* w, const float* w_s, void* y_bf16, int64_t M,
                    int64_t N, int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of fp32 workspace bfp8_gemm would use at this shape: split-K of a
 * skinny problem, or the split last round of a large one (0 when neither
 * applies).  Pure host function (the plan assumes the 256 CUs of MI355X). */
size_t bfp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/* Grouped fp8_gemm over one GPU's share of routed experts ([BT] "MoE trace":
 * each local expert with tokens runs expert(x[idx]); [PY] "Honest Limits":
 * a fused grouped GEMM replaces the per-expert Python loop).
 * Rows [off[g], off[g+1]) of a belong to expert g and are multiplied by its
 * weight b[g]:
 *     c[r, n] = bf16_rne( sum_kb P_kb[r, n] * a_s[r, kb] * b_s[g, n/128, kb] )
 *   a     : e4m3 [total_M, K] rows sorted by group       a_s : fp32 [total_M, K/128]
 *   b     : e4m3 [G, N, K]                               b_s : fp32 [G, ceil(N/128), K/128]
 *   c_bf16: bf16 [total_M, N] output
 *   group_offsets : DEVICE int32 [G+1], normally off[0] = 0 and
 *     off[g] <= off[g+1] <= total_M.  Empty groups are allowed, and off[G] may
 *     be less than total_M, so total_M can be a capacity (e.g. the offsets
 *     written by bfp8_moe_dispatch, read by the kernel without a host copy).
 *     The kernel clamps every offset into [0, total_M] and each group's end to
 *     at least its start, so no offset value makes it read or write outside
 *     the buffers.  Rows outside every group are never written.
 * Errors: as bfp8_gemm, plus BFP8_ERR_GROUPS if G < 1. */
int bfp8_gemm_grouped(const void* a, const float* a_s, const void* b, const float* b_s,
                      void* c_bf16, const int32_t* group_offsets, int32_t G,
                      int64_t total_M, int64_t N, int64_t K, void* stream);

/* The BF16 branch of linear() ([PY] "FP8 with per-block scales": the weight
 * is expanded to bf16 by weight_dequant and multiplied by an ordinary BF16
 * matmul).  C = A * B^T with B a Linear weight (out_features x in_features):
 *     c[m, n] = bf16_rne( sum_k a[m, k] * b[n, k] )      (fp32 accumulation)
 *   a_bf16 : bf16 [M, K], 16-byte aligned
 *   b_bf16 : bf16 [N, K], 16-byte aligned (e.g. bfp8_weight_dequant's output)
 *   c_bf16 : bf16 [M, N] output, 2-byte aligned
 *   workspace : optional fp32 scratch for large problems (K >= 80 * 128) whose
 *     last round of 256 x 256 tiles is at most half full: those tiles run as two
 *     K halves into it, then one ordered reduction.  NULL: every tile runs its
 *     whole K range.  If non-NULL it must hold bfp8_gemm_bf16_workspace_size
 *     (M, N, K) bytes and be 16-byte aligned; its contents do not matter.
 * Errors: BFP8_ERR_SHAPE if M < 0, N < 0, K <= 0, K % 64 != 0 or K >= 2^22;
 * BFP8_ERR_NULL; BFP8_ERR_ALIGN; BFP8_ERR_WORKSPACE (workspace too small). */
int bfp8_gemm_bf16(const void* a_bf16, const void* b_bf16, void* c_bf16, int64_t M, int64_t N,
                   int64_t K, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of fp32 workspace bfp8_gemm_bf16 would use at this shape (0 when its
 * last round is not split).  Pure host function (planned for 256 CUs). */
size_t bfp8_gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K);

/* ----------------------------------------------------------------------
 * MoE dispatch and combine around the grouped GEMM ([BT] "MoE trace": per
 * expert counts; for each local expert with tokens, the tokens routed to it,
 * in ascending order, go through the expert, and y[idx] gains the expert's
 * output times the routing weight, y starting at zero; [DF] expert sharding:
 * a GPU holds the contiguous expert range expert_lo .. expert_lo + G - 1).
 * Together: bfp8_moe_dispatch -> bfp8_act_quant_rows -> bfp8_gemm_grouped ->
 * bfp8_moe_combine, all on the device, with no host synchronization.
 * ---------------------------------------------------------------------- */

/* Bytes of int32 workspace bfp8_moe_dispatch needs (a multiple of 16; 0 when
 * T * k == 0).  Pure host function. */
size_t bfp8_moe_dispatch_workspace_size(int64_t T, int32_t k, int32_t G);

/* Stable counting sort of the routed (token, slot) pairs by local expert.
 *   topk_idx      : DEVICE int32 [T, k] expert id of each (token, slot); ids
 *                   outside expert_lo .. expert_lo + G - 1 are not local
 *   group_offsets : DEVICE int32 [G+1] output: rows of local expert g are
 *                   off[g] .. off[g+1]; off[0] = 0, off[G] = local pairs
 *   row_token     : DEVICE int32 [T * k] output: row_token[r] = token of row r
 *                   for r < off[G] (entries past off[G] are not written)
 *   slot_row      : DEVICE int32 [T, k] output: the row of each (token, slot),
 *                   or -1 when the slot's expert is not local
 * Inside one expert, rows follow (token, slot) order, so tokens ascend, as in
 * the pages' per-expert selection.  Deterministic.
 *   workspace     : DEVICE, at least bfp8_moe_dispatch_workspace_size(T, k, G)
 *                   bytes, 4-byte aligned; contents on entry are ignored.
 * T == 0 still writes group_offsets (all zero).
 * Errors: BFP8_ERR_SHAPE if T < 0, k < 1 or T * k >= 2^31; BFP8_ERR_GROUPS if
 * G < 1 or G > BFP8_MOE_MAX_GROUPS; BFP8_ERR_NULL for a NULL pointer that the
 * call needs; BFP8_ERR_ALIGN if an int32 array or the workspace is not 4-byte
 * aligned; BFP8_ERR_WORKSPACE if workspace_bytes is too small. */
int bfp8_moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t expert_lo,
                      int32_t G, int32_t* group_offsets, int32_t* row_token, int32_t* slot_row,
                      void* workspace, size_t workspace_bytes, void* stream);

/* act_quant of gathered rows: for r < min(*num_rows, M) output row r is
 * act_quant of input row row_token[r] (same arithmetic as bfp8_act_quant,
 * bit for bit; quantization is row-local, so this equals gathering rows of
 * act_quant(x)).  Rows past min(*num_rows, M), and rows whose token is
 * outside [0, T), are not written.
 *   x_bf16    : bf16 [T, K], 16-byte aligned
 *   row_token : DEVICE int32 [M]
 *   num_rows  : DEVICE int32 [1], e.g. group_offsets + G of bfp8_moe_dispatch;
 *               NULL means M rows
 *   q_e4m3    : e4m3 [M, K] output, 16-byte aligned
 *   scales    : fp32 [M, K/128] output
 * Errors: BFP8_ERR_SHAPE if T < 0, M < 0, K <= 0 or K % 128 != 0;
 * BFP8_ERR_NULL; BFP8_ERR_ALIGN. */
int bfp8_act_quant_rows(const void* x_bf16, int64_t T, const int32_t* row_token,
                        const int32_t* num_rows, void* q_e4m3, float* scales, int64_t M,
                        int64_t K, void* stream);

/* Weighted combine of the expert outputs back to token order:
 *     y[t, n] = bf16_rne( sum_{j < k, 0 <= slot_row[t,j] < rows} weights[t, j] *
 *                         expert_out[slot_row[t, j], n] )
 * summed in fp32 in slot order (fused multiply-adds); a token with no local
 * slot gets zeros.  This is the pages' y[idx] += expert(x[idx]) * weight over
 * the local experts, with one rounding to bf16 at the end instead of one per
 * expert.
 *   expert_out_bf16 : bf16 [rows, N] (the grouped GEMM's output)
 *   slot_row        : DEVICE int32 [T, k] (from bfp8_moe_dispatch)
 *   weights         : DEVICE fp32 [T, k] routing weights
 *   y_bf16          : bf16 [T, N] output (every element written)
 * A 16-byte vector kernel runs when N % 8 == 0 and expert_out and y are
 * 16-byte aligned; a scalar one otherwise.
 * Errors: BFP8_ERR_SHAPE if T < 0, k < 1, N < 0, rows < 0, T > 2^24,
 * T * k >= 2^31 or N > 65535 * 2048; BFP8_ERR_NULL;
 * BFP8_ERR_ALIGN if a bf16 pointer is not 2-byte or an int32/fp32 pointer not
 * 4-byte aligned. */
int bfp8_moe_combine(const void* expert_out_bf16, int64_t rows, const int32_t* slot_row,
                     const float* weights, void* y_bf16, int64_t T, int32_t k, int64_t N,
                     void* stream);

/* Test helper: encodes the 2^32 float32 bit patterns first .. first+count-1
 * to e4m3 codes with the same device routine act_quant uses (variant 0), or
 * with the alternative routine (variant 1), into out[count] (device).
 * Lets a test compare the device encoder with the oracle on every input.
 * Errors: BFP8_ERR_NULL, BFP8_ERR_SHAPE (count < 0 or first+count > 2^32),
 * BFP8_ERR_ARG (unknown variant). */
int bfp8_e4m3_encode_range(uint32_t first, int64_t count, void* out, int variant, void* stream);

/* Test helper: rounds the float32 bit patterns first .. first+count-1 to
 * bf16 with the device routine the dequant kernel and the GEMM epilogue use
 * (variant 0) or with the alternative bit-level routine (variant 1), into
 * out[count] (device, uint16 bf16 bit patterns, 2-byte aligned).
 * Errors: BFP8_ERR_NULL, BFP8_ERR_SHAPE, BFP8_ERR_ALIGN, BFP8_ERR_ARG. */
int bfp8_bf16_round_range(uint32_t first, int64_t count, void* out, int variant, void* stream);

/* Introspection helper: the name of the kernel configuration bfp8_gemm uses
 * for an M x N x K problem on the current device (static storage; "none" for
 * a shape bfp8_gemm would reject or skip).  Lets tests and benchmarks record
 * which tile configuration ran. */
const char* bfp8_gemm_kernel_name(int64_t M, int64_t N, int64_t K);

/* Human-readable name of a status code (static storage). */
const char* bfp8_status_string(int status);

/* BFP8_VERSION of the built library. */
int bfp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BFP8_H */
