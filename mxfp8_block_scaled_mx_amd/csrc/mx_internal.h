// Internal declarations shared by the host API and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp8.h"

namespace mx {

constexpr int kMaxGroups = MX_MAX_GROUPS;

// Row groups of a quantize call (kernel argument, passed by value).
struct QuantGroups {
  int32_t n;                        // number of groups (>= 1)
  int32_t row0[kMaxGroups + 1];     // first row of group g
  int32_t pcol0[kMaxGroups + 1];    // first column of group g in the columnwise layout
  int32_t tile0[kMaxGroups + 1];    // first row-tile of group g (prefix of ceil(m_g/128))
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
  QuantGroups groups;
};

// Launch the quantize kernel (arguments already validated).
hipError_t launch_quantize(const QuantArgs& args, int x_dtype, int total_row_tiles, hipStream_t stream);
constexpr int kQuantTileRows = 128;
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
  int32_t tile0[kMaxGroups + 1];
  int32_t gid[kMaxGroups];
  int32_t a0[kMaxGroups];
  int32_t len[kMaxGroups];
  int32_t pc0[kMaxGroups];          // first column of the group in columnwise layouts
};

struct GemmArgs {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  void* c;
  int64_t lda, ldb, ldc;
  int64_t b_group_stride;           // codes; scales use b_group_stride/32
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
  float* dprobs_part;               // bwd: [n_tiles_n, R] partial sums
  int32_t R;                        // rows of the routed activations
  GemmGroups groups;
};

hipError_t launch_gemm(int mode, int epi, bool scale_dword, const GemmArgs& args, int total_tiles,
                       hipStream_t stream);

hipError_t launch_dprobs_reduce(const float* part, float* dprobs, int32_t R, int32_t n_parts,
                                hipStream_t stream);

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTileK = 128;

}  // namespace mx
