/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) MXFP8 block-scaled grouped-MLP library.
 *
 * What the library computes (the pages this follows):
 *   - MXFP8: 8-bit E4M3 values with one power-of-two (E8M0) scale per block of
 *     32 consecutive values ("Efficient MoE training for biological foundation
 *     models", section "Key technical approaches in the recipe", item 2; the
 *     TransformerEngine Llama 3 recipe page, section "MXFP8 vs BF16 throughput
 *     on Llama-3.1": MXFP8BlockScaling with E4M3).
 *   - GroupedLinear: one grouped GEMM over per-expert row counts (split_sizes)
 *     instead of one launch per expert (same article, item 1).
 *   - GroupedLinear -> ScaledSwiGLU -> GroupedLinear fused into one forward op
 *     and one backward op, with the SwiGLU activation and routing-weight
 *     scaling fused and 16-bit master weights quantized each step (same
 *     article, item 3).
 *
 * Number formats and rounding (readings of what the pages leave open):
 *   - block scale exponent e = floor(log2(amax)) - 8, clamped to [-127, 127];
 *     E8M0 scale code = e + 127 (0x00 for an all-zero block);
 *   - element code = E4M3 (bias 7, no infinities) of v / 2^e by
 *     round-to-nearest-even, saturating at +-448 (never NaN), subnormals kept,
 *     sign bit copied from the input (so -0.0 and negative underflow -> 0x80).
 *   - Non-finite inputs are outside the contract: outputs are unspecified.
 *
 * Layouts (all row-major, "ld" = elements between consecutive rows):
 *   - rowwise MXFP8 of a [rows, cols] matrix: codes uint8 [rows, cols] and
 *     scales uint8 [rows, cols/32]; block j of row r covers columns
 *     [32j, 32j+32). cols must be a multiple of 32.
 *   - columnwise MXFP8 = rowwise MXFP8 of the transpose: codes [cols, P],
 *     scales [cols, P/32]. With row groups (split_sizes), group g's rows are
 *     zero-padded to P_g = ceil(m_g/32)*32 and occupy columns
 *     [sum_{j<g} P_j, + P_g); blocks never straddle groups; padding codes are
 *     0x00. Without groups, P = ceil(rows/32)*32.
 *   - The scale matrix of a code matrix with leading dimension ld has leading
 *     dimension ld/32, and a code offset o (whose column part is a multiple of
 *     32) corresponds to scale offset o/32.
 *   - Weights are [out, in]: W1 [E, 2F, H] (gate rows 0..F-1, up rows F..2F-1),
 *     W2 [E, H, F]; no biases. bf16 arrays are raw IEEE bfloat16 bit patterns.
 *
 * Conventions for every entry point:
 *   - Device pointers unless marked "host". The caller owns all memory; the
 *     library never allocates, frees or keeps device memory between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronizing. split_sizes are host arrays.
 *     grouped_mlp_bwd also runs its wgrad stages on a side
 *     stream the library creates per thread and device (on first use, default
 *     priority, kept until the process ends): it waits on an event recorded on
 *     `stream` and `stream` waits on an event recorded after the side work,
 *     so to the caller all work is ordered on `stream` (also under graph
 *     capture). `stream` must belong to the current device.
 *   - Arguments are validated before anything is enqueued. On any non-OK
 *     status nothing was enqueued and no output was touched; mx_last_error()
 *     then holds a one-line description (thread-local).
 *   - No C++ exception crosses this boundary. Calls on different streams may
 *     run concurrently; calls that write the same buffers must be ordered by
 *     the caller.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MX_API __attribute__((visibility("default")))
#else
#define MX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_EINVAL = 1,       /* null pointer, bad enum value, inconsistent flags */
  MX_ESHAPE = 2,       /* sizes inconsistent or not multiples of 32 */
  MX_EALIGN = 3,       /* pointer or leading dimension misaligned */
  MX_EWORKSPACE = 4,   /* workspace or saved buffer smaller than required */
  MX_EHIP = 5,         /* a HIP runtime call failed (text in mx_last_error) */
  MX_EUNSUPPORTED = 6  /* valid request this build does not support */
} mx_status;

typedef enum mx_dtype { MX_BF16 = 0, MX_F32 = 1 } mx_dtype;

typedef enum mx_group_mode {
  MX_GROUP_M = 0, /* groups split the rows of A (fprop, dgrad) */
  MX_GROUP_K = 1  /* groups split the K dimension (wgrad) */
} mx_group_mode;

/* Largest number of groups (experts) one call accepts. */
#define MX_MAX_GROUPS 128

/* Name of a status code (static string). */
MX_API const char* mx_status_string(int status);

/* Text of the last non-OK status returned on this thread ("" if none). */
MX_API const char* mx_last_error(void);

/* Library ABI version: 1. */
MX_API int mx_version(void);

/*
 * mx_device_copy -- a plain device-to-device copy of `bytes` bytes (a
 * multiple of 16; dst and src 16-byte aligned, not overlapping), enqueued on
 * `stream`. It is the measured HBM reference for the memory-bound casts (the
 * same read-then-write traffic without the arithmetic), not part of the MLP.
 * Errors: MX_ESHAPE, MX_EINVAL (null pointer), MX_EALIGN, MX_EHIP.
 */
MX_API mx_status mx_device_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * mx_quantize -- MXFP8 quantization of a [rows, cols] matrix (row-major,
 * contiguous, ld = cols) into the rowwise and/or columnwise layouts.
 *
 * Follows the block-scaling definition above (article item 2).
 *   x            bf16 or f32 input [rows, cols], 16-byte aligned.
 *   x_dtype      MX_BF16 or MX_F32.
 *   rows, cols   rows >= 0, cols > 0 and cols % 32 == 0.
 *   group_sizes  host int64[num_groups] row counts (>= 0) summing to rows, or
 *                NULL with num_groups == 0 for a single group of all rows.
 *                Groups only change the columnwise layout.
 *   q_row,s_row  rowwise codes [rows, cols] (16-byte aligned) and scales
 *                [rows, cols/32]; both NULL to skip the rowwise copy.
 *   q_col,s_col  columnwise codes [cols, sumP] (16-byte aligned) and scales
 *                [cols, sumP/32]; both NULL to skip the columnwise copy.
 * At least one copy must be requested. Errors: MX_EINVAL (null x, both copies
 * skipped, half of a pair given, bad dtype), MX_ESHAPE (cols % 32, negative or
 * inconsistent sizes), MX_EALIGN, MX_EUNSUPPORTED (num_groups > MX_MAX_GROUPS).
 */
MX_API mx_status mx_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                      const int64_t* group_sizes, int32_t num_groups,
                      uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                      void* stream);

/*
 * mx_grouped_gemm -- grouped block-scaled GEMM  C = A . B^T  on MXFP8 operands
 * (GroupedLinear over split_sizes, article item 1; MXFP8 operands, item 2).
 * Both operands are K-contiguous rowwise MXFP8 (codes + scales); products are
 * accumulated in fp32.
 *
 * mode = MX_GROUP_M (fprop/dgrad): sizes[g] rows of A belong to group g (in
 *   order, sum = M); group g uses B_g = b + g*b_group_stride (codes, [N, ldb])
 *   and b_scale + g*b_group_stride/32; C is [M, ldc].
 * mode = MX_GROUP_K (wgrad): sizes[g] are unpadded row counts; group g
 *   contracts over columns [sum_{j<g} P_j, + P_g) of A [M, lda] and B [N, ldb]
 *   (the columnwise-grouped layout, K = sum P); C_g = c + g*c_group_stride is
 *   [M, ldc]; a group with sizes[g] == 0 writes zeros (accumulate = 0) or
 *   leaves C_g unchanged (accumulate = 1).
 *
 *   a, a_scale   A codes [M, lda] and scales [M, lda/32]; lda % 32 == 0.
 *   b, b_scale   B codes [N, ldb] (per group in MX_GROUP_M) and scales.
 *   c            output, c_dtype MX_F32 or MX_BF16 (round to nearest even).
 *   accumulate   1: C += result (MX_F32 only); 0: C = result.
 * Requirements: K % 32 == 0, N % 32 == 0, K <= lda, K <= ldb, N <= ldc,
 * b_group_stride % 32 == 0, a/b 16-byte aligned, c 16-byte aligned and
 * ldc % 4 == 0, 1 <= num_groups <= MX_MAX_GROUPS.
 */
MX_API mx_status mx_grouped_gemm(int32_t mode, int32_t num_groups, const int64_t* sizes,
                          int64_t M, int64_t N, int64_t K,
                          const uint8_t* a, const uint8_t* a_scale, int64_t lda,
                          const uint8_t* b, const uint8_t* b_scale, int64_t ldb,
                          int64_t b_group_stride,
                          void* c, int32_t c_dtype, int64_t ldc, int64_t c_group_stride,
                          int32_t accumulate, void* stream);

/* Shape of one grouped MLP call: R routed rows, E experts, hidden H, ffn F. */
typedef struct mx_mlp_dims {
  int32_t num_experts;
  int64_t rows;
  int64_t hidden;
  int64_t ffn;
} mx_mlp_dims;

/*
 * grouped_mlp_sizes -- byte sizes of the caller-provided buffers for one
 * shape and split: fwd_workspace (scratch of grouped_mlp_fwd), saved (what
 * grouped_mlp_fwd keeps for grouped_mlp_bwd in training) and bwd_workspace
 * (scratch of grouped_mlp_bwd). Any output pointer may be NULL.
 * Errors: MX_EINVAL, MX_ESHAPE (H or F not multiples of 128, split mismatch).
 */
MX_API mx_status grouped_mlp_sizes(const mx_mlp_dims* dims, const int64_t* split_sizes,
                            size_t* fwd_workspace, size_t* saved, size_t* bwd_workspace);

/*
 * grouped_mlp_intermediates -- where the fused ops leave the intermediates
 * they requantize inside the call: A = w*silu(g)*u of the forward epilogue
 * and dH1 = [dg | du] of the backward epilogue (the intermediates the fused
 * op keeps out of HBM in bf16/fp32 form, article item 3), plus the saved H1.
 * All values are byte offsets into the buffers of one call with the same
 * dims and split_sizes; they are valid after the call that writes them and
 * until the buffer is reused:
 *   forward workspace:  A rowwise codes [R, F] and scales;
 *   saved:              H1 bf16 [R, 2F], A columnwise codes [F, sumP] and scales;
 *   backward workspace: dH1 rowwise codes [R, 2F] and scales, dH1 columnwise
 *                       codes [2F, sumP] and scales.
 * Codes are in the public layouts above. Scales are k-tiled: the scales of a
 * [rows, K] code matrix split K into steps of 128 columns numbered q, and
 * the four block scales of row r in step q are the bytes
 *     ((r / 32) * nq + q) * 128 + (r % 32) * 4 + {0, 1, 2, 3};
 * rowwise: q = column / 128, nq = K / 128 (rows padded to a multiple of 32);
 * columnwise: expert e's padded rows P_e are its own steps starting at
 * q0_e = sum_{e' < e} ceil(P_e' / 128), nq = nq_col = q0_E, and the bytes of
 * blocks past P_e in its last step are unspecified.
 * Errors: as grouped_mlp_sizes; MX_EINVAL if out is NULL.
 */
typedef struct mx_mlp_intermediates {
  size_t a_row_codes, a_row_scales;                        /* forward workspace */
  size_t h1, a_col_codes, a_col_scales;                    /* saved */
  size_t dh1_row_codes, dh1_row_scales, dh1_col_codes, dh1_col_scales;  /* backward workspace */
  int64_t nq_col;
} mx_mlp_intermediates;
MX_API mx_status grouped_mlp_intermediates(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                           mx_mlp_intermediates* out);

/*
 * grouped_mlp_fwd -- fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear
 * forward (article item 3). For expert e and its rows X_e (routing weight w
 * per row):
 *     H1 = Xq_e . W1q_e^T;  g = H1[:, :F], u = H1[:, F:];
 *     A  = w * silu(g) * u  (fp32, formed before requantization);
 *     Y  = Aq . W2q_e^T     (bf16, round to nearest even)
 * where Xq, W1q, W2q, Aq are rowwise MXFP8 copies made inside the call (the
 * bf16 master weights are quantized on every call).
 *   split_sizes  host int64[E], >= 0, sum = R; rows are ordered by expert.
 *   x            bf16 [R, H];  probs f32 [R] routing weights (NULL = all 1).
 *   w1, w2       bf16 [E, 2F, H] and [E, H, F].
 *   y            bf16 [R, H] output.
 *   saved        NULL for inference; otherwise a buffer of `saved` bytes
 *                (grouped_mlp_sizes) that receives H1 (bf16), the columnwise
 *                copies of X, A, W1, W2 for grouped_mlp_bwd.
 *   workspace    fwd_workspace bytes of scratch, 256-byte aligned.
 * Requires H % 128 == 0 and F % 128 == 0 (the internal MXFP8 copies keep
 * their scales in 128-column steps), 1 <= E <= MX_MAX_GROUPS. All pointers
 * 16-byte aligned. The layout of the workspace and saved buffers is private
 * to the library.
 */
MX_API mx_status grouped_mlp_fwd(const mx_mlp_dims* dims, const int64_t* split_sizes,
                          const void* x, const float* probs, const void* w1, const void* w2,
                          void* y, void* saved, size_t saved_bytes,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * grouped_mlp_bwd -- the corresponding fused backward op (article item 3),
 * straight-through for quantization; every GEMM runs on MXFP8 copies:
 *     dA  = dYq_row . colwise(W2_e)          (K = H)
 *     dg  = dA*w*u*s*(1 + g*(1-s)), du = dA*w*silu(g), s = sigmoid(g),
 *           with g, u from the saved bf16 H1;  dprobs = sum_f dA*silu(g)*u
 *     dX  = dH1q_row . colwise(W1_e)         (K = 2F, bf16 out)
 *     dW2_e (+)= colwise(dY_e)^T . colwise(A_e)    (fp32)
 *     dW1_e (+)= colwise(dH1_e)^T . colwise(X_e)   (fp32)
 *   dy           bf16 [R, H];  probs as in the forward (NULL = all 1).
 *   saved        the buffer filled by grouped_mlp_fwd with the same inputs.
 *   dx           bf16 [R, H] output.
 *   dprobs       f32 [R] output, or NULL to skip.
 *   dw1, dw2     f32 [E, 2F, H] and [E, H, F]; accumulate_wgrad = 1 adds into
 *                them (fp32 main-grad), 0 overwrites. An expert with no rows
 *                leaves its dW unchanged (1) or zero (0).
 *   workspace    bwd_workspace bytes of scratch.
 */
MX_API mx_status grouped_mlp_bwd(const mx_mlp_dims* dims, const int64_t* split_sizes,
                          const void* dy, const float* probs, const void* saved, size_t saved_bytes,
                          void* dx, float* dprobs, float* dw1, float* dw2, int32_t accumulate_wgrad,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cached MXFP8 weights ("quantized initialization" in the Llama 3 recipe
 * page's MXFP8 throughput section, and the 16-bit master weights of item 3 of
 * the MoE article): the two weight casts of grouped_mlp_fwd are taken out of
 * the step. A training loop quantizes its bf16 master weights once after each
 * optimizer update and runs every forward and backward of that step on the
 * cached copies, which hold exactly the codes and scales grouped_mlp_fwd
 * would have made from the same weights, so results are identical.
 *
 * grouped_mlp_weight_cache_bytes -- size of the cache for E, H, F (rows and
 * split are not used). Errors: MX_EINVAL, MX_ESHAPE as grouped_mlp_sizes.
 *
 * grouped_mlp_quantize_weights -- cast w1 bf16 [E, 2F, H] and w2 bf16
 * [E, H, F] into `cache` (caller-owned device buffer, 256-byte aligned, at
 * least grouped_mlp_weight_cache_bytes), rowwise and columnwise. Async on
 * `stream`. The cache layout is private to the library; it stays valid until
 * the caller overwrites or frees it. Errors: MX_EINVAL (null pointers),
 * MX_EALIGN, MX_EWORKSPACE (cache too small), MX_EHIP.
 *
 * grouped_mlp_fwd_cached / grouped_mlp_bwd_cached -- grouped_mlp_fwd and
 * grouped_mlp_bwd with the weights read from a filled cache instead of being
 * cast from bf16. Same arguments, buffer sizes and errors otherwise; a
 * `saved` buffer written by grouped_mlp_fwd_cached holds no weight copies and
 * must be consumed by grouped_mlp_bwd_cached with the same cache.
 */
MX_API mx_status grouped_mlp_weight_cache_bytes(const mx_mlp_dims* dims, size_t* bytes);
MX_API mx_status grouped_mlp_quantize_weights(const mx_mlp_dims* dims, const void* w1, const void* w2,
                                              void* cache, size_t cache_bytes, void* stream);
MX_API mx_status grouped_mlp_fwd_cached(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                        const void* x, const float* probs, const void* cache,
                                        size_t cache_bytes, void* y, void* saved, size_t saved_bytes,
                                        void* workspace, size_t workspace_bytes, void* stream);
MX_API mx_status grouped_mlp_bwd_cached(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                        const void* dy, const float* probs, const void* cache,
                                        size_t cache_bytes, const void* saved, size_t saved_bytes,
                                        void* dx, float* dprobs, float* dw1, float* dw2,
                                        int32_t accumulate_wgrad, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Token dispatch and combine around the grouped MLP. Each token activates
 * `topk` experts ("Efficient MoE training for biological foundation
 * models", Dense vs. MoE scaling), and GroupedLinear takes each expert's
 * input tokens gathered into one group with per-expert counts, split_sizes
 * (Key technical approaches, item 1). These calls build that grouping on the
 * device.
 *
 * mx_moe_dispatch_workspace_bytes -- scratch bytes of mx_moe_dispatch
 * (0 for invalid sizes).
 *
 * mx_moe_dispatch -- routed rows ordered by expert, then token.
 *   x          bf16 [tokens, hidden], hidden % 8 == 0.
 *   topk_idx   int32 [tokens, topk]: the experts of each token (distinct per
 *              token). An entry outside [0, num_experts) is dropped: its perm
 *              is -1 and it takes no routed row.
 *   topk_w     f32 [tokens, topk] routing weights, or NULL (then probs_perm
 *              must be NULL too).
 *   x_perm     bf16 [tokens * topk, hidden]: routed row r holds the row of its
 *              token. Only the first sum(counts) rows are written. x and
 *              x_perm may both be NULL: routing only, no row copy (for
 *              grouped_mlp_fwd_gather, which reads the token rows itself).
 *   probs_perm f32 [tokens * topk]: routing weight of each routed row.
 *   perm       int32 [tokens, topk]: routed row of entry (t, j), or -1.
 *   row_token  int32 [tokens * topk]: token of each routed row.
 *   counts     int64 [num_experts]: rows per expert (split_sizes; copy them to
 *              the host for grouped_mlp_fwd).
 *   workspace  at least mx_moe_dispatch_workspace_bytes, 4-byte aligned.
 * The result is deterministic: no global atomics. With tokens == 0 only
 * counts (set to 0) and workspace are used; the other pointers may be NULL.
 * Errors: MX_EINVAL, MX_ESHAPE, MX_EALIGN (x, x_perm 16-byte), MX_EWORKSPACE,
 * MX_EUNSUPPORTED (num_experts > MX_MAX_GROUPS, tokens * topk >= 2^31).
 *
 * mx_moe_combine -- y[t] = sum over the token's slots j with perm[t, j] >= 0
 * of y_perm[perm[t, j]]. The sum is fp32 in slot order, rounded once to bf16
 * (nearest even). The routing weights were applied inside the MLP, so the sum
 * is unweighted. perm must come from mx_moe_dispatch with the same tokens and
 * topk, and y_perm must hold at least that call's routed rows.
 *   y_perm bf16 [>= sum(counts), hidden]; y bf16 [tokens, hidden].
 */
/*
 * mx_quantize_fp4 -- MXFP4 cast of a bf16 [rows, cols] tensor. MX
 * block scaling at 4 bits, the format of the MI355X mxfp4 runs on the ROCm
 * Megatron page ("examples/llama: default-on fusion & DP-comm perf toggles"),
 * following the OCP MX rules as for MXFP8. Each 32-value block along a row
 * gets an E8M0 scale 2^e with e = floor(log2 amax) - 2, clamped to
 * [-127, 127]. Each element becomes the nearest E2M1 value (0, 0.5, 1, 1.5,
 * 2, 3, 4, 6 and negatives) of v / 2^e, ties to the even code, saturating at
 * 6, with the sign of v kept.
 *   q      uint8 [rows, cols/2]: rowwise codes, two per byte, element 2i in
 *          the low nibble.
 *   s      uint8 [rows, cols/32]: rowwise scale codes, row-major.
 *   q_col  uint8 [cols, rows/2]: columnwise codes (rowwise of the transpose).
 *   s_col  uint8 [cols, rows/32]: columnwise scale codes.
 * Either pair may be NULL (not both). Requires cols % 32 == 0, and
 * rows % 32 == 0 for the columnwise pair; x, q, q_col 16-byte aligned.
 * Non-finite inputs are outside the contract. Errors: MX_EINVAL, MX_ESHAPE,
 * MX_EALIGN, MX_EUNSUPPORTED.
 */
MX_API mx_status mx_quantize_fp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                                 uint8_t* q_col, uint8_t* s_col, void* stream);

/*
 * mx_gemm_fp4 -- C[m, n] = A[m, k] . B[n, k]^T on MXFP4 operands, the GEMM of
 * the 4-bit MX runs (same page as mx_quantize_fp4), on the scaled MFMA with
 * E2M1 operands: element value = E2M1(code) * 2^(scale code - 127), products
 * summed in fp32.
 *   a, a_s  uint8 [m, k/2] codes and uint8 [m, k/32] scales (the rowwise
 *           layout of mx_quantize_fp4: element 2i in the low nibble);
 *   b, b_s  the same for B [n, k];
 *   c       [m, n] row-major, bf16 (rounded to nearest even) or fp32 per
 *           c_dtype; written, never read.
 * Caller-owned device memory; nothing is allocated. Requires k a positive
 * multiple of 64 (at most 2^24); a, b, c 16-byte aligned. m or n zero is a
 * no-op. Errors: MX_EINVAL, MX_ESHAPE, MX_EALIGN, MX_EUNSUPPORTED, MX_EHIP.
 */
MX_API mx_status mx_gemm_fp4(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s, int64_t m,
                             int64_t n, int64_t k, void* c, mx_dtype c_dtype, void* stream);

/*
 * mx_grouped_gemm_fp4 -- the grouped (GroupedLinear) form of mx_gemm_fp4 over
 * per-expert split_sizes ("Efficient MoE training for biological foundation
 * models", Key technical approaches item 1): the rows of A are split into
 * `groups` consecutive groups of group_sizes[g] rows, and the rows of group g
 * get C = A_g . B_g^T.
 *   a, a_s       rowwise MXFP4 A [sum(group_sizes), k] (codes, scales);
 *   b, b_s       rowwise MXFP4 weights, groups x [n, k], group after group
 *                (codes [groups, n, k/2], scales [groups, n, k/32]);
 *   group_sizes  host int64 [groups], each >= 0 (empty groups allowed);
 *   c            [sum(group_sizes), n] row-major, bf16 or fp32 per c_dtype.
 * 1 <= groups <= MX_MAX_GROUPS. Same requirements, ownership and errors as
 * mx_gemm_fp4, which is this call with one group.
 */
MX_API mx_status mx_grouped_gemm_fp4(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                     const int64_t* group_sizes, int32_t groups, int64_t n, int64_t k, void* c,
                                     mx_dtype c_dtype, void* stream);

/*
 * NVFP4 -- the 4-bit recipe the Llama 3 recipe page lists beside FP8 and
 * MXFP8 ("TransformerEngine-accelerated Llama 3 training with native PyTorch
 * training loop", Supported Models and Training Features, and Quantized
 * Training), and whose first and last layers the MI355X recipe keeps in BF16
 * ("examples/llama: default-on fusion & DP-comm perf toggles - #141",
 * Changes). The pages name the format but not its arithmetic; this library
 * implements its published form: E2M1 elements in blocks of 16 values with
 * one E4M3 scale per block and one fp32 scale per tensor. In fp32 arithmetic
 * rounded to nearest:
 *     S   = 2688 / amax (448 * 6; 1 for amax = 0; at most 2^64)
 *     s_b = E4M3 code of (bmax / 6) * S, saturating at 448
 *     q   = E2M1 code of x * (S / E4M3(s_b)) (nearest, ties to even,
 *           saturating at 6, sign kept; 0 / 0x8 when s_b = 0)
 * and an element's value is E2M1(q) * E4M3(s_b) / S.
 *
 * mx_quantize_nvfp4 -- x bf16 [rows, cols] (contiguous, cols % 16 == 0):
 *   amax   device fp32, receives max |x| of the whole tensor (the call
 *          reduces it first; NULL is an error);
 *   q, s   rowwise codes [rows, cols/2] (two per byte, low nibble first) and
 *          E4M3 scale codes [rows, cols/16]; or both NULL;
 *   q_col, s_col  the columnwise copy (rowwise copy of the transpose, blocks
 *          of 16 rows; rows % 16 == 0) [cols, rows/2] and [cols, rows/16];
 *          or both NULL. Both copies use the same S.
 * Errors: MX_ESHAPE, MX_EINVAL (no output, half a layout, null x or amax),
 * MX_EALIGN (x 16-byte, q/q_col 8-byte, amax 4-byte), MX_EUNSUPPORTED,
 * MX_EHIP.
 *
 * mx_gemm_nvfp4 / mx_grouped_gemm_nvfp4 -- C = A . B^T (grouped: group g's
 * rows of A times its weight B_g^T) with NVFP4 operands in the rowwise layout
 * of mx_quantize_nvfp4, A's tensor amax at a_amax and B_g's at b_amax[g]
 * (device fp32; one per group). gfx950's scaled MFMA takes power-of-two
 * (E8M0) scales per 32 values only, so NVFP4 runs on the fp16 MFMA: every
 * element times its E4M3 block scale is exact in fp16 and is formed in
 * registers; sums are fp32; the product of the two 1/S factors is applied
 * once to each result (one fp32 rounding). k must be a positive multiple of
 * 128 (at most 2^24); scales 8-byte aligned; other requirements, outputs and
 * errors as mx_gemm_fp4 / mx_grouped_gemm_fp4.
 */
MX_API mx_status mx_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s,
                                   uint8_t* q_col, uint8_t* s_col, float* amax, void* stream);
MX_API mx_status mx_gemm_nvfp4(const uint8_t* a, const uint8_t* a_s, const float* a_amax, const uint8_t* b,
                               const uint8_t* b_s, const float* b_amax, int64_t m, int64_t n, int64_t k, void* c,
                               mx_dtype c_dtype, void* stream);
MX_API mx_status mx_grouped_gemm_nvfp4(const uint8_t* a, const uint8_t* a_s, const float* a_amax, const uint8_t* b,
                                       const uint8_t* b_s, const float* b_amax, const int64_t* group_sizes,
                                       int32_t groups, int64_t n, int64_t k, void* c, mx_dtype c_dtype,
                                       void* stream);

/*
 * MXFP4 MLP -- the grouped MLP of grouped_mlp_fwd / grouped_mlp_bwd with
 * every GEMM on MXFP4 copies (E2M1 elements, one E8M0 scale per 32 values;
 * as mx_quantize_fp4) instead of MXFP8: the MLP of a layer assigned to FP4
 * ("TransformerEngine-accelerated Llama 3 training with native PyTorch
 * training loop", Layer-Wise Precision; the mxfp4 runs of "examples/llama:
 * default-on fusion & DP-comm perf toggles - #141", which put every layer in
 * FP4). Same formulas, straight-through backward and argument meanings as
 * grouped_mlp_fwd / grouped_mlp_bwd:
 *     H1 = Xq . W1q^T (fp32);  A = w * silu(g) * u (fp32), requantized;
 *     Y  = Aq . W2q^T (bf16);
 *     dA = dYq . colwise(W2) (fp32);  dH1 = [dg | du] from the bf16 H1;
 *     dX = dH1q . colwise(W1) (bf16);  dW2_e, dW1_e (+)= fp32 group-K products
 * of the per-expert columnwise copies (mx_quantize_fp4_colwise_grouped's
 * layout). The bf16 master weights are quantized on every forward call.
 *
 * grouped_mlp_fp4_sizes -- byte sizes of the forward workspace, the saved
 * buffer and the backward workspace for one shape and split (any output
 * pointer may be NULL). Same dims and split requirements as
 * grouped_mlp_sizes (H, F multiples of 128, 1 <= E <= MX_MAX_GROUPS, split
 * summing to R); the padded rows sum P must stay at or below 2^24.
 * grouped_mlp_fwd_fp4 -- x bf16 [R, H], probs f32 [R] (NULL = all 1), w1 bf16
 * [E, 2F, H], w2 bf16 [E, H, F], y bf16 [R, H]; saved NULL for inference.
 * grouped_mlp_bwd_fp4 -- dy bf16 [R, H], saved from grouped_mlp_fwd_fp4 with
 * the same inputs, dx bf16 [R, H], dprobs f32 [R] or NULL, dw1 f32 [E, 2F, H]
 * and dw2 f32 [E, H, F] (accumulate_wgrad != 0 adds into them).
 * Buffers are caller-owned; x, w, y, dy, dx, dw 16-byte aligned, workspace and
 * saved 256-byte aligned; their layouts are private to the library.
 * Errors: as grouped_mlp_fwd / grouped_mlp_bwd (MX_EINVAL, MX_ESHAPE,
 * MX_EALIGN, MX_EWORKSPACE, MX_EUNSUPPORTED, MX_EHIP).
 */
MX_API mx_status grouped_mlp_fp4_sizes(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                       size_t* fwd_workspace, size_t* saved, size_t* bwd_workspace);
MX_API mx_status grouped_mlp_fwd_fp4(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                     const void* x, const float* probs, const void* w1, const void* w2,
                                     void* y, void* saved, size_t saved_bytes,
                                     void* workspace, size_t workspace_bytes, void* stream);
MX_API mx_status grouped_mlp_bwd_fp4(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                     const void* dy, const float* probs, const void* saved, size_t saved_bytes,
                                     void* dx, float* dprobs, float* dw1, float* dw2, int32_t accumulate_wgrad,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cached MXFP4 weights: the cached-weight form of the MXFP4 MLP, as
 * grouped_mlp_quantize_weights / grouped_mlp_fwd_cached / grouped_mlp_bwd_cached
 * are for the MXFP8 MLP (quantized initialization of the Llama 3 recipe
 * page's MXFP8 throughput section, applied to the 4-bit layer of its
 * Layer-Wise Precision section). The per-expert weight casts of
 * grouped_mlp_fwd_fp4 leave the step: a training loop casts its bf16 master
 * weights once after each optimizer update and runs forward and backward on
 * the cached copies, which hold exactly the codes and scales
 * grouped_mlp_fwd_fp4 would make from the same weights, so the results are
 * bit-identical.
 *
 * grouped_mlp_fp4_weight_cache_bytes -- size of the cache for E, H, F (rows
 * and split are not used; the other dims rules of grouped_mlp_fp4_sizes hold).
 * grouped_mlp_fp4_quantize_weights -- cast w1 bf16 [E, 2F, H] and w2 bf16
 * [E, H, F] into `cache` (caller-owned device buffer, 256-byte aligned, at
 * least grouped_mlp_fp4_weight_cache_bytes), rowwise and each expert's
 * columnwise copy. Async on `stream`. The cache layout is private to the
 * library; it stays valid until the weights change. Errors: MX_EINVAL,
 * MX_ESHAPE, MX_EALIGN, MX_EWORKSPACE (cache too small), MX_EHIP.
 * grouped_mlp_fwd_fp4_cached / grouped_mlp_bwd_fp4_cached --
 * grouped_mlp_fwd_fp4 and grouped_mlp_bwd_fp4 with the weights read from a
 * filled cache instead of being cast; same workspace and saved sizes
 * (grouped_mlp_fp4_sizes) and errors, plus the cache checks above. The saved
 * buffer written by grouped_mlp_fwd_fp4_cached holds no weight copies and must
 * be consumed by grouped_mlp_bwd_fp4_cached with the same cache.
 */
MX_API mx_status grouped_mlp_fp4_weight_cache_bytes(const mx_mlp_dims* dims, size_t* bytes);
MX_API mx_status grouped_mlp_fp4_quantize_weights(const mx_mlp_dims* dims, const void* w1, const void* w2,
                                                  void* cache, size_t cache_bytes, void* stream);
MX_API mx_status grouped_mlp_fwd_fp4_cached(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                            const void* x, const float* probs, const void* cache,
                                            size_t cache_bytes, void* y, void* saved, size_t saved_bytes,
                                            void* workspace, size_t workspace_bytes, void* stream);
MX_API mx_status grouped_mlp_bwd_fp4_cached(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                            const void* dy, const float* probs, const void* cache,
                                            size_t cache_bytes, const void* saved, size_t saved_bytes,
                                            void* dx, float* dprobs, float* dw1, float* dw2,
                                            int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * mx_quantize_fp4_colwise_grouped -- columnwise MXFP4 of a routed activation
 * with per-expert padding, the layout of the 4-bit weight gradient (the
 * MXFP4 form of the grouped columnwise MXFP8 layout above; MXFP4 as in
 * mx_quantize_fp4): the rows of x (bf16 [rows, cols], contiguous) are split
 * into `groups` consecutive groups of group_sizes[g] rows; each group's rows
 * are zero-padded to P_g = a multiple of 32 and, transposed, quantized in
 * blocks of 32 along the rows.
 *   q_col  codes [cols, sum P_g / 2] (two per byte, low nibble first),
 *          group g at bytes [sum_{g'<g} P_g' / 2, + P_g / 2) of every row;
 *   s_col  E8M0 scales [cols, sum P_g / 32].
 * Every byte of both outputs is written (padding rows give code 0).
 * Errors: MX_ESHAPE (cols not a positive multiple of 32, negative sizes or
 * sizes not summing to rows), MX_EINVAL (groups outside 1..MX_MAX_GROUPS,
 * null pointers), MX_EALIGN (x or q_col not 16-byte aligned),
 * MX_EUNSUPPORTED (too large), MX_EHIP.
 *
 * mx_grouped_gemm_fp4_wgrad -- the weight-gradient (group-K) GEMM at MXFP4
 * with fp32 accumulation into a main gradient:
 *   C_g (+)= A[:, K_g] . B[:, K_g]^T   for every group g,
 * K_g = group g's padded range [sum_{g'<g} P_g', + P_g) of the contraction
 * (P_g = group_sizes[g] rounded up to a multiple of 32), with A [m, K] and
 * B [n, K] (K = sum P_g) in the layout mx_quantize_fp4_colwise_grouped
 * writes (codes [m, K/2], scales [m, K/32]; likewise B). Elements are
 * E2M1(code) * 2^(scale - 127) and the products are exact; the sums are fp32
 * on the scaled MFMA. c is fp32 [groups, m, n] (group g at c + g*m*n,
 * row-major); accumulate != 0 adds into it (a group with no rows leaves its
 * C_g unchanged), else C_g is overwritten (zeros for a group with no rows).
 * The ROCm MI355X recipe notes that its 4-bit wgrad GEMM emits BF16 only,
 * which breaks fp32 main-gradient accumulation ("examples/llama: default-on
 * fusion & DP-comm perf toggles - #141", the GRAD_REDUCE_IN_BF16 guard);
 * this call is that fp32-accumulating form.
 * Errors: MX_EINVAL (groups outside 1..MX_MAX_GROUPS, null pointers),
 * MX_ESHAPE (negative sizes), MX_EALIGN (a, b, c not 16-byte aligned),
 * MX_EUNSUPPORTED (K above 2^24 or too many tiles), MX_EHIP.
 */
MX_API mx_status mx_quantize_fp4_colwise_grouped(const void* x, int64_t rows, int64_t cols,
                                                 const int64_t* group_sizes, int32_t groups,
                                                 uint8_t* q_col, uint8_t* s_col, void* stream);
MX_API mx_status mx_grouped_gemm_fp4_wgrad(const uint8_t* a, const uint8_t* a_s, const uint8_t* b,
                                           const uint8_t* b_s, const int64_t* group_sizes, int32_t groups,
                                           int64_t m, int64_t n, float* c, int32_t accumulate,
                                           void* stream);

MX_API size_t mx_moe_dispatch_workspace_bytes(int64_t tokens, int32_t topk, int32_t num_experts);

/*
 * grouped_mlp_bwd_gather -- grouped_mlp_bwd with dY read the same way: routed
 * row r of dY is row row_token[r] of dy_tokens (bf16 [tokens, hidden]), the
 * gradient of the combine (each token's output is the sum of its routed
 * rows, so every routed row receives its token's output gradient). dx is
 * per routed row ([rows, hidden]); mx_moe_combine sums it per token (the
 * gradient of the dispatch). Same buffers, results and errors as
 * grouped_mlp_bwd with dy = dy_tokens[row_token].
 *
 * grouped_mlp_fwd_gather -- grouped_mlp_fwd with the token gather fused into
 * the cast of X: routed row r is row row_token[r] of x_tokens (bf16
 * [tokens, hidden]), read by the MXFP8 quantize itself, so the routed bf16
 * copy of X is never written. row_token is device int32 [rows], as
 * mx_moe_dispatch returns it, and split_sizes are that call's counts. An
 * index outside [0, tokens) reads as a zero row. Everything else, including
 * buffer sizes, `saved` for grouped_mlp_bwd, results and errors, is as for
 * grouped_mlp_fwd, with x = x_tokens[row_token]. The backward's dX is per
 * routed row; mx_moe_combine sums it back per token.
 */
MX_API mx_status grouped_mlp_bwd_gather(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                        const void* dy_tokens, int64_t tokens,
                                        const int32_t* row_token, const float* probs,
                                        const void* saved, size_t saved_bytes, void* dx,
                                        float* dprobs, float* dw1, float* dw2,
                                        int32_t accumulate_wgrad, void* workspace,
                                        size_t workspace_bytes, void* stream);
MX_API mx_status grouped_mlp_fwd_gather(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                        const void* x_tokens, int64_t tokens,
                                        const int32_t* row_token, const float* probs,
                                        const void* w1, const void* w2, void* y, void* saved,
                                        size_t saved_bytes, void* workspace,
                                        size_t workspace_bytes, void* stream);
MX_API mx_status mx_moe_dispatch(const void* x, const int32_t* topk_idx, const float* topk_w,
                                 int64_t tokens, int64_t hidden, int32_t topk, int32_t num_experts,
                                 void* x_perm, float* probs_perm, int32_t* perm, int32_t* row_token,
                                 int64_t* counts, void* workspace, size_t workspace_bytes,
                                 void* stream);
MX_API mx_status mx_moe_combine(const void* y_perm, const int32_t* perm, int64_t tokens,
                                int64_t hidden, int32_t topk, void* y, void* stream);

/*
 * Device-resident split_sizes (sync-free). GroupedLinear takes the per-expert
 * row counts, split_sizes ("Efficient MoE training for biological foundation
 * models", Key technical approaches item 1); when they are produced on the
 * GPU, for example as mx_moe_dispatch's counts, these calls read them there:
 * the call's first kernel turns them into the group tables of every cast and
 * GEMM of the call, so the host never copies them back nor waits for them,
 * and the counts may still be in flight on `stream` when the call is made.
 *
 * grouped_mlp_sizes_device_split -- buffer sizes (bytes) for the two calls
 * below, valid for every split of dims->rows routed rows over the experts:
 * the columnwise copies and their k-tiled scales are laid out for the
 * largest padded total any split can reach (rows + 31 * min(experts, rows)
 * columns), and each workspace holds the device-built tables. These layouts
 * are not those of grouped_mlp_sizes: `saved` of grouped_mlp_fwd_device_split
 * is read by grouped_mlp_bwd_device_split only.
 *
 * grouped_mlp_fwd_device_split -- grouped_mlp_fwd (article item 3) with
 *   split_sizes  device int64 [num_experts], read when the call's first
 *                kernel runs (stream order). Expert e owns routed rows
 *                [sum_{e'<e} m_e', + m_e). The counts are clamped on the
 *                device: a negative count reads as 0, and a count that would
 *                take the running sum past dims->rows is cut there (later
 *                experts get no rows). The clamped sum S may be below
 *                dims->rows, as when the dispatch drops entries: routed rows
 *                S .. rows-1 are not read, and their rows of y are not
 *                written.
 *   row_token    optional gather as in grouped_mlp_fwd_gather (routed row r
 *                is row row_token[r] of x, which has `tokens` rows); null:
 *                x is the routed rows [rows, hidden] and tokens is ignored.
 *   cache        optional weight cache of grouped_mlp_quantize_weights; null:
 *                the weights are cast from w1, w2 inside the call (as
 *                grouped_mlp_fwd); given: w1 and w2 are not read.
 * Results for the first S rows are those of grouped_mlp_fwd (or _gather /
 * _cached) on the clamped split, except that no split-K tail is used, so
 * GEMM2 may sum a tile's k range in another order.
 * Errors: as grouped_mlp_fwd; MX_EINVAL for a null split_sizes, MX_EALIGN if
 * it is not 8-byte aligned. A count's value is never an error.
 *
 * grouped_mlp_bwd_device_split -- the corresponding backward, with the same
 * split_sizes (the same values the forward read), optional row_token gather
 * of dY as in grouped_mlp_bwd_gather, and optional weight cache (null: the
 * columnwise weight copies that the forward left in `saved`). Rows S ..
 * rows-1 of dx are not written and dprobs is 0 there; dw1 / dw2 of experts
 * with no rows are zeroed (accumulate_wgrad == 0) or left as they are.
 * Errors as grouped_mlp_bwd, plus those of split_sizes above.
 */
MX_API mx_status grouped_mlp_sizes_device_split(const mx_mlp_dims* dims, size_t* fwd_workspace,
                                                size_t* saved, size_t* bwd_workspace);
MX_API mx_status grouped_mlp_fwd_device_split(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                              const void* x, int64_t tokens, const int32_t* row_token,
                                              const float* probs, const void* w1, const void* w2,
                                              const void* cache, size_t cache_bytes, void* y,
                                              void* saved, size_t saved_bytes, void* workspace,
                                              size_t workspace_bytes, void* stream);
MX_API mx_status grouped_mlp_bwd_device_split(const mx_mlp_dims* dims, const int64_t* split_sizes,
                                              const void* dy, int64_t tokens, const int32_t* row_token,
                                              const float* probs, const void* cache, size_t cache_bytes,
                                              const void* saved, size_t saved_bytes, void* dx,
                                              float* dprobs, float* dw1, float* dw2,
                                              int32_t accumulate_wgrad, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * mx_moe_dispatch_noalloc -- mx_moe_dispatch for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments and results without
 * the workspace. Its scratch (the per-block expert histograms and row bases)
 * is a library-owned array of 65536 int32 (256 KiB) per GPU, created with the
 * library's device code and held until the process ends; the call allocates
 * nothing. The caller still provides every input and output.
 *   Limit: ceil(tokens * topk / 256) * num_experts + 1 <= 65536 (for example
 *   16384 tokens, top-2 of 128 experts); larger requests return
 *   MX_EUNSUPPORTED and enqueue nothing.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, different threads) race and must be ordered by
 * the caller. The array needs no clearing between calls. Other errors as
 * mx_moe_dispatch; MX_EHIP if the array's device address cannot be found.
 */
MX_API mx_status mx_moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, const float* topk_w,
                                         int64_t tokens, int64_t hidden, int32_t topk,
                                         int32_t num_experts, void* x_perm, float* probs_perm,
                                         int32_t* perm, int32_t* row_token, int64_t* counts,
                                         void* stream);

/*
 * mx_set_stage_events -- optional per-stage timing of the fused MLP calls
 * (observability only; the results are the same). While events are set, the
 * fused MLP calls run every stage on the caller's stream in order, without
 * the side stream, so each stage's time is its own. events points to
 * `count` hipEvent_t handles owned by the caller, or is NULL to switch timing
 * off. While set on the calling thread, grouped_mlp_fwd records events[i] on
 * its stream before stage i and after the last stage (stages: quantize X,
 * quantize W1, quantize W2, GEMM1 + SwiGLU epilogue, GEMM2 -> 6 events) and
 * grouped_mlp_bwd does the same for its stages (quantize dY, dgrad2 + SwiGLU
 * backward epilogue, dprobs reduction, wgrad2, dgrad1, wgrad1 -> 7 events).
 * Events beyond `count` are not recorded. Errors: MX_EINVAL (count < 0, or
 * count > 0 with events NULL).
 */
MX_API mx_status mx_set_stage_events(void* const* events, int32_t count);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H */
