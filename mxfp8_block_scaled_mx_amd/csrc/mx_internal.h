// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp8.h"

namespace mx {

constexpr int kMaxGroups = MX_MAX_GROUPS;

// Two layouts of the E8M0 scales of a code matrix [rows, K]:
//  - row-major: byte (r, b) at r * (K/32) + b (the public layout);
//  - k-tiled: K is cut into groups (the columnwise layouts' per-expert
//    segments; one group for a rowwise matrix), each group into steps of 128
//    columns (4 blocks) numbered q = q0(group) + b_local/4 over all groups
//    (nq steps in total), and byte (r, b) sits at
//      ((r >> 5) * nq + q) * 128 + (r & 31) * 4 + b_local % 4,
//    so the scales of 32 consecutive rows for one 128-column step are one
//    contiguous 128-byte line. Bytes of blocks past a group's end in its last
//    step are unspecified.
// Scale address generator used by the kernels for one operand:
//   step word of row r, step q = (r >> 5) * grp + (r & 31) * row + q * step.
struct ScaleStrides {
  int64_t grp;                      // bytes per 32-row group
  int32_t row;                      // bytes per row inside a group
  int32_t step;                     // bytes per 128-column step
};
inline ScaleStrides row_major_scales(int64_t ld) { return {32 * (ld / 32), (int32_t)(ld / 32), 4}; }
inline ScaleStrides k_tiled_scales(int64_t nq) { return {nq * 128, 4, 128}; }

// Row groups of a quantize call (kernel argument, passed by value).
struct QuantGroups {
  int32_t n;                        // number of groups (>= 1)
  int32_t row0[kMaxGroups + 1];     // first row of group g
  int32_t pcol0[kMaxGroups + 1];    // first column of group g in the columnwise layout
  int32_t tile0[kMaxGroups + 1];    // first row-tile of group g (prefix of ceil(m_g/128))
  int32_t q0[kMaxGroups + 1];       // k-tiled columnwise scales: first 128-column step of group g
};

struct QuantArgs {
  const void* x;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
  int64_t cols;
  int64_t ld_col;                   // leading dimension of the columnwise codes (sum P)
  int32_t n_col_tiles;
  int32_t tiled;                    // scales in the k-tiled layout (both copies)
  int32_t nq_row;                   // k-tiled rowwise scales: cols / 128
  int32_t nq_col;                   // k-tiled columnwise scales: steps over all groups
  int32_t rows;                     // total rows (k-tiled rowwise: pad rows up to a multiple of 32 get 0)
  // optional gather: row r of the (routed) input is row row_index[r] of x,
  // which has index_rows rows; an index outside [0, index_rows) reads zeros
  const int32_t* row_index;
  int32_t index_rows;
  QuantGroups groups;
  // non-null: the group table lives in device memory (built there from
  // per-group sizes held on the device) and replaces `groups`; the grid is
  // sized for the worst case and row tiles past the table's last one exit
  const QuantGroups* groups_dev;
};

// Launch the quantize kernel (arguments already validated).
hipError_t launch_quantize(const QuantArgs& args, int x_dtype, int total_row_tiles, hipStream_t stream);
constexpr int kQuantTileRows = 128;
// Plain device copy of `bytes` (a multiple of 16; 16-byte aligned pointers).
hipError_t launch_device_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);
inline int quant_tile_cols(int x_dtype) { return x_dtype == MX_BF16 ? 128 : 64; }

// Epilogues of the grouped GEMM.
enum GemmEpi : int {
  EPI_F32 = 0,         // C (+)= acc, fp32
  EPI_BF16 = 1,        // C = bf16(acc)
  EPI_SWIGLU_FWD = 2,  // A = w*silu(g)*u -> rowwise/columnwise MXFP8, H1 -> bf16
  EPI_SWIGLU_BWD = 3   // SwiGLU backward on dA -> dH1 MXFP8 (both layouts), dprobs partials
};

// Per-group tile table (kernel argument). Slot s is processed in order; a0/len
// are (first row, rows) in MX_GROUP_M and (first K column, padded K) in MX_GROUP_K.
struct GemmGroups {
  int32_t n;
  // MX_GROUP_K with every slot holding the same number of tiles, a multiple
  // of 32: chunks of 32 tile ids rotate over the slots (see locate_tile)
  int32_t interleave;
  int32_t tile0[kMaxGroups + 1];
  int32_t gid[kMaxGroups];
  int32_t a0[kMaxGroups];
  int32_t len[kMaxGroups];
  int32_t pc0[kMaxGroups];          // first column of the group in columnwise layouts
  int32_t q0[kMaxGroups];           // first 128-column step of the group in k-tiled scales
};

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  void* c;
  int64_t lda, ldb, ldc;
  int64_t b_group_stride;           // codes of consecutive B groups (MX_GROUP_M)
  int64_t bs_group_stride;          // scales of consecutive B groups (MX_GROUP_M)
  ScaleStrides sa, sb;              // scale addressing of A and B
  int32_t k_tiled;                  // scales k-tiled (MX_GROUP_K: steps from groups.q0)
  int64_t as_bytes, bs_bytes;       // extent of the A and B scale arrays
  int64_t c_group_stride;
  int32_t M;                        // rows of C in MX_GROUP_K (A rows)
  int32_t N;                        // columns of C (B rows); SwiGLU fwd: 2F
  int32_t K;                        // MX_GROUP_M contraction length
  int32_t n_tiles_n;                // tiles along N
  int32_t accumulate;
  // fused epilogues
  int32_t F;                        // ffn size
  int64_t ld_col;                   // columnwise layouts: sum of padded group rows
  const float* probs;               // routing weights [R] or null (= 1)
  uint16_t* h1;                     // fwd: saved H1 bf16 [R, 2F] (may be null); bwd: input
  uint8_t* q_row;                   // fwd: A rowwise [R, F]; bwd: dH1 rowwise [R, 2F]
  uint8_t* s_row;
  uint8_t* q_col;                   // fwd: A columnwise [F, ld_col]; bwd: dH1 [2F, ld_col]
  uint8_t* s_col;
  int32_t nq_row;                   // k-tiled epilogue scales: steps of the rowwise output
  int32_t nq_col;                   // k-tiled epilogue scales: steps of the columnwise output
  float* dprobs_part;               // bwd: [n_tiles_n, R] partial sums
  int32_t R;                        // rows of the routed activations
  // split-K tail (MX_GROUP_M, plain epilogues): workgroups past split_f each
  // take 1/split_s of the k-steps of tile split_f + (wg - split_f) / split_s
  // and write an fp32 partial tile to split_ws; split_s <= 1: no split
  int32_t split_f, split_s;
  float* split_ws;
  GemmGroups groups;
  // non-null: the group table lives in device memory and replaces `groups`
  // (k-tiled scales only, no split-K tail); the grid is sized for the worst
  // case and workgroups past the table's tile count exit
  const GemmGroups* groups_dev;
};

hipError_t launch_gemm(int mode, int epi, bool scale_dword, const GemmArgs& args, int total_tiles,
                       hipStream_t stream);

// Sum the split-K partials of the tail tiles into C (after launch_gemm).
hipError_t launch_split_reduce(int epi, const GemmArgs& args, int tail_tiles, hipStream_t stream);
// Split-K tail bounds: at most this many tail tiles, each in at most this many parts.
constexpr int kMaxSplitTiles = 128;
constexpr int kMaxSplitParts = 4;

// dprobs[r] = sum of the n_parts partials of row r; with rows_dev, rows at
// or past *rows_dev are written 0.
hipError_t launch_dprobs_reduce(const float* part, float* dprobs, int32_t R, int32_t n_parts,
                                const int32_t* rows_dev, hipStream_t stream);

// Group tables of the fused MLP built on the device from per-expert row
// counts held in device memory (no host round trip). The counts are clamped:
// a negative count reads as 0 and a count that would take the running sum
// past R is cut there, so every table stays inside the buffers sized for R
// rows.
struct MlpDevPlan {
  int32_t rows;                     // sum of the clamped counts (<= R)
  int32_t pad_;
  QuantGroups act;                  // activation row groups (X, dY casts)
  GemmGroups m[3];                  // group-M tables, one per n-tile count below
  GemmGroups k[2];                  // group-K tables, one per tile count per slot below
};
struct MlpDevPlanArgs {
  const int64_t* counts;            // [E] device
  MlpDevPlan* plan;                 // device, written
  int32_t E, R;
  int32_t m_tiles_n[3];             // n-tiles per m-tile of each group-M table
  int32_t k_slot_tiles[2];          // tiles per slot of each group-K table
  int32_t k_interleave[2];          // interleave flag of each group-K table
};
hipError_t launch_mlp_dev_plan(const MlpDevPlanArgs& args, hipStream_t stream);

// Token dispatch / combine around the grouped MLP (mx_moe.hip).
constexpr int kMoeBlock = 256;      // entries per workgroup in the counting passes
struct MoeDispatchArgs {
  const void* x;                    // bf16 [tokens, hidden]
  const int32_t* topk_idx;          // [tokens, topk]
  const float* topk_w;              // [tokens, topk] or null
  int64_t tokens, hidden;
  int32_t topk, experts;
  void* x_perm;                     // bf16 [tokens * topk, hidden]
  float* probs_perm;                // [tokens * topk] or null
  int32_t* perm;                    // [tokens, topk]
  int32_t* row_token;               // [tokens * topk]
  int64_t* counts;                  // [experts]
  int32_t* workspace;               // ceil(tokens * topk / kMoeBlock) * experts + 1 int32
};
hipError_t launch_moe_dispatch(const MoeDispatchArgs& args, hipStream_t stream);
// Device address of the current device's dispatch scratch array (looked up
// once per device).
constexpr int64_t kDispatchScratchWords = 1 << 16;
hipError_t dispatch_scratch(int32_t** out);
hipError_t launch_moe_combine(const void* y_perm, const int32_t* perm, int64_t tokens, int64_t hidden, int32_t topk,
                              void* y, hipStream_t stream);

// Rowwise MXFP4 cast (mx_fp4.hip).
hipError_t launch_quantize_fp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                               uint8_t* s_col, hipStream_t stream);
// MXFP4 grouped GEMM C_g = A_g . B_g^T (mx_fp4.hip): kFp4GemmTileM x
// kFp4GemmTileN tiles, m-tiles restarting at each group; c_f32 selects fp32
// (else bf16) output.
constexpr int kFp4GemmTileM = 256, kFp4GemmTileN = 256;
struct Fp4Groups {
  int32_t n;                         // groups
  int32_t tile0[kMaxGroups + 1];     // first m-tile of group g; tile0[n] = all m-tiles
  int64_t row0[kMaxGroups + 1];      // first row of group g; row0[n] = M
};
// Split-K tail: the tiles from id `first` on (the last, partial round) each
// run as `parts` workgroups over consecutive k-tile ranges, writing fp32
// partial tiles (kFp4GemmTileM x kFp4GemmTileN, row-major, unit
// (id - first) * parts + part) to ws; a reduce kernel adds each tile's parts
// in part order and writes C. parts <= 1: no split.
struct Fp4Split {
  int32_t first, parts;
  float* ws;
};
hipError_t launch_gemm_fp4(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           const Fp4Groups& gr, int64_t N, int64_t K, void* c, int32_t c_f32, hipStream_t stream,
                           const Fp4Split& split = Fp4Split{0, 0, nullptr});
// Groups of the columnwise MXFP4 cast: group g's rows [row0[g], row0[g+1]),
// padded to a multiple of 32 at columns [pcol0[g], pcol0[g+1]) of the
// result; its 128-row tiles are tile0[g] .. tile0[g+1] - 1.
struct Fp4ColGroups {
  int32_t n;
  int32_t tile0[kMaxGroups + 1];
  int64_t row0[kMaxGroups + 1];
  int64_t pcol0[kMaxGroups + 1];
};
// ScaledSwiGLU of the MXFP4 MLP fused into the columnwise cast: the values
// cast are formed on the fly instead of read. Forward: A = w * silu(g) * u
// [R, F] from GEMM1's fp32 H1 = [g | u] [R, 2F], H1 written in bf16 to h1_out
// (or not, when null). Backward: dH1 = [dg | du] [R, 2F] from dgrad2's fp32
// dA [R, F] and the saved bf16 H1, and per-row partial sums of dprobs
// (sum over f of dA * silu(g) * u) to dprobs_part [F / 64, R] (summed by
// launch_dprobs_reduce). probs null means routing weights 1.
struct Fp4SwigluArgs {
  const float* h1f;          // forward: H1 [R, 2F] fp32
  uint16_t* h1_out;          // forward: H1 [R, 2F] bf16 (or null)
  const float* da;           // backward: dA [R, F] fp32
  const uint16_t* h1;        // backward: saved H1 [R, 2F] bf16
  float* dprobs_part;        // backward: [F / 64, R] (or null)
  const float* probs;        // [R] or null
  int64_t R, F;
};
hipError_t launch_swiglu_fp4_cast(bool backward, const Fp4SwigluArgs& sw, const Fp4ColGroups& gr, uint8_t* q_col,
                                  uint8_t* s_col, uint8_t* q_row, uint8_t* s_row, hipStream_t stream);
// x is bf16 or (x_f32) fp32 [rows, cols]; q_row / s_row (or null) receive the
// rowwise copy of the same pass.
hipError_t launch_quantize_fp4_grouped(const void* x, bool x_f32, int64_t rows, int64_t cols, const Fp4ColGroups& gr,
                                       uint8_t* q_col, uint8_t* s_col, uint8_t* q_row, uint8_t* s_row,
                                       hipStream_t stream);
// NVFP4 (mx_fp4.hip): the cast writes the tensor amax to *amax (device fp32)
// and rowwise codes [rows, cols/2] + E4M3 scales [rows, cols/16] and/or the
// columnwise pair [cols, rows/2] + [cols, rows/16]; cols % 16 == 0 (rows % 16
// for the columnwise copy). The grouped GEMM is launch_gemm_fp4's with NVFP4
// operands (K % 128 == 0), the tensor scale of A from *a_amax and of group g's
// weight from b_amax[g].
hipError_t launch_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                                 uint8_t* s_col, float* amax, hipStream_t stream);
hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* as, const float* a_amax, const uint8_t* b,
                             const uint8_t* bs, const float* b_amax, const Fp4Groups& gr, int64_t N, int64_t K,
                             void* c, int32_t c_f32, hipStream_t stream);
// ScaledSwiGLU forward of the MXFP4 MLP at inference (mx_fp4.hip): H1 fp32
// [R, 2F] -> A's rowwise MXFP4 copy [R, F/2] + [R, F/32]; F % 32 == 0; probs
// null = all 1. (Training runs launch_swiglu_fp4_cast.)
hipError_t launch_swiglu_fwd_fp4(const float* h1f, const float* probs, int64_t R, int64_t F, uint8_t* aq, uint8_t* as,
                                 hipStream_t stream);
// MXFP4 group-K product C_g (+)= A[:, K_g] . B[:, K_g]^T (fp32), K_g =
// [k0[g], k0[g+1]) in values (multiples of 32): A [M, k0[n]] and B
// [N, k0[n]] rowwise-packed MXFP4 (the columnwise layouts of two routed
// activations); C_g at c + g * M * N, row-major [M, N].
struct Fp4KGroups {
  int32_t n;
  int64_t k0[kMaxGroups + 1];
};
hipError_t launch_gemm_fp4_group_k(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                   const Fp4KGroups& gr, int64_t M, int64_t N, float* c, int32_t accumulate,
                                   hipStream_t stream);

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileK = 128;

}  // namespace mx
