// Rowwise MXFP4 cast: E2M1 elements with one E8M0 scale per 32 consecutive
// values (the MX block format the pages name next to MXFP8, run at 4 bits on
// MI355X: "examples/llama: default-on fusion & DP-comm perf toggles", the
// mxfp4 Llama runs). Scale exponent floor(log2 amax) - 2 (2 = exponent of
// E2M1's largest value, 6); element = nearest E2M1 value of v / 2^e, ties to
// the even code, saturating at 6; two codes per byte, element 2i in the low
// nibble.
//
// Rowwise: one thread per 32-value block: four 16-byte loads, a local amax,
// the scale code from the amax exponent bits, the elements divided by 2^e and
// rounded by the hardware's scaled E2M1 convert, 16 bytes of codes stored at
// once. Columnwise: see the columnwise kernel. HBM-bound.
#include <algorithm>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// E2M1 codes of 8 values, value i in nibble i of the word. The scaled convert
// (v_cvt_scalef32_pk_fp4_*) divides each value by 2^E, E the exponent field
// of `scale` read as an E8M0 code (so code 0 means 2^-127), rounds to the
// nearest E2M1 value with ties to the even code (the midpoints 0.25, 0.75,
// 1.25, 1.75, 2.5, 3.5 and 5 go to the neighbour whose code is even),
// saturates at 6 and keeps the sign of zero. Checked on hardware against that
// rule written out: every bf16 value under scale codes 0..253, every tie point
// and its neighbouring fp32 values at scale 1, signed zeros and values whose
// quotient is an fp32 subnormal, both operand positions; NaN inputs differ
// and lie outside the casts' contract.
__device__ __forceinline__ float e8m0_as_scale(uint32_t code) { return __uint_as_float(code << 23); }
__device__ __forceinline__ uint32_t e2m1x8(const float* v, float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
  return w;
}
// the same for 8 bf16 values as loaded (value 2i in the low half of dword i)
__device__ __forceinline__ uint32_t e2m1x8_bf16(const uint4& raw, float scale) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, raw.x), scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, raw.y), scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, raw.z), scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2, raw.w), scale, 3);
  return w;
}

// One 32-value MXFP4 block: scale code (floor(log2 amax) - 2 + 127 = biased
// exponent - 2, clamped at 0 for a zero or subnormal amax or a biased
// exponent below 3) and the 16 code bytes, element 2i in the low nibble.
__device__ __forceinline__ uint32_t fp4_block(const float (&v)[32], uint4& codes) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = umax(am, abs_bits(v[i]));
  const uint32_t eb = am >> 23;
  const uint32_t sc = eb > 2u ? eb - 2u : 0u;
  const float scale = e8m0_as_scale(sc);
  codes = make_uint4(e2m1x8(&v[0], scale), e2m1x8(&v[8], scale), e2m1x8(&v[16], scale), e2m1x8(&v[24], scale));
  return sc;
}

__global__ __launch_bounds__(256) void quantize_fp4_rowwise_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                   uint8_t* q, uint8_t* s) {
  const int64_t nb = cols / 32;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= rows * nb) return;
  const int64_t r = blk / nb, b = blk - r * nb;
  const uint4* src = reinterpret_cast<const uint4*>(x + r * cols + b * 32);
  uint4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = src[i];
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[8 * i + 0] = bf16_lo(raw[i].x); v[8 * i + 1] = bf16_hi(raw[i].x);
    v[8 * i + 2] = bf16_lo(raw[i].y); v[8 * i + 3] = bf16_hi(raw[i].y);
    v[8 * i + 4] = bf16_lo(raw[i].z); v[8 * i + 5] = bf16_hi(raw[i].z);
    v[8 * i + 6] = bf16_lo(raw[i].w); v[8 * i + 7] = bf16_hi(raw[i].w);
  }
  uint4 codes;
  const uint32_t sc = fp4_block(v, codes);
  *reinterpret_cast<uint4*>(q + r * (cols / 2) + b * 16) = codes;
  s[r * nb + b] = (uint8_t)sc;
}

// Columnwise MXFP4 (= rowwise of the transpose): codes [cols, ldp/2] and
// scales [cols, ldp/32]; with q_row given, the rowwise pair [rows, cols/2] +
// [rows, cols/32] from the same read of x. Grouped (per-expert) columnwise
// layout: row tiles restart at each group's first row, rows past the group's
// end read as zeros, and group g's padded rows land at columns
// [pcol0[g], + pad32(m_g)) of the result. One group of all rows is the plain
// columnwise cast. T is the input type: bf16 bits (uint16_t) or fp32 (the
// fp32 intermediates of the MXFP4 MLP).
//
// Tile: 128 rows x 256 bytes (128 bf16 or 64 fp32 columns), 256 threads.
// Thread t issues its 8 row pieces (row 16 p + t / 16, 16-byte chunk t % 16)
// first; the rowwise copy comes from registers (the 4 or 8 threads of a
// 32-block reduce its amax with xor shuffles; one scale word per row and
// tile). The tile is staged in LDS unchanged; thread t then reads 32 dwords
// down rows 32 (t / 64) .. + 31 (one or two columns), forms each column's
// block, and the codes are staged as [column][64 bytes] (16-byte piece j of
// column c at piece j ^ ((c >> 2) & 3), spreading the writes over the banks)
// and leave as each column's 64-byte run of the tile's 128 rows.
// Order: a 128-byte output line holds 256 values, two tiles' worth in both
// layouts, so tile ids pair consecutive row tiles inside each column tile
// (id = 2 (row pair) n_ct + 2 ct + (row tile & 1)) and go to the XCDs in
// chunks of 64: the two halves of every line are written by workgroups that
// run at the same time on the same XCD and meet in its L2.
// SRC: where the values come from -- the input x, or (T = float) the
// ScaledSwiGLU forward or backward formed from Fp4SwigluArgs (the fused
// MXFP4 MLP; cols = F resp. 2F). A 64-column tile of the backward lies wholly
// in the dg half (columns below F) or the du half, F being a multiple of 128.
enum Fp4Src : int { kSrcX = 0, kSrcSwigluFwd = 1, kSrcSwigluBwd = 2 };
constexpr int kFp4ColTileRows = 128, kFp4CastChunk = 64;
// routing weight 1, read where a cast has no probs (so that the weight loads
// stay unconditional)
__device__ const float kUnitWeight = 1.0f;

template <typename T, int SRC = kSrcX>
__global__ __launch_bounds__(256) void quantize_fp4_colwise_kernel(const T* x, int64_t rows, int64_t cols,
                                                                   uint8_t* q, uint8_t* s, uint8_t* q_row,
                                                                   uint8_t* s_row, Fp4ColGroups gr, int64_t ldp,
                                                                   Fp4SwigluArgs sw) {
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int VPT = 16 / (int)sizeof(T);   // values per 16-byte chunk
  constexpr int TC = 16 * VPT;               // tile columns
  constexpr int TR = kFp4ColTileRows;
  constexpr int TPB = 32 / VPT;              // threads per 32-block along a row
  constexpr int NB = TC / 32;                // 32-blocks per tile row
  constexpr int CPS = kBf16 ? 2 : 1;         // columns per dword
  // the input tile as loaded, then (once every column is in registers) the
  // columnwise codes [column][64 bytes]
  __shared__ __attribute__((aligned(16))) uint8_t tile[TR * 256];
  __shared__ uint32_t cs_t[TC];              // columnwise scale bytes [column][block]
  static_assert(TC * 64 <= TR * 256, "columnwise staging must fit the input tile");

  // column tiles of the grid: the SwiGLU backward covers the dg half (columns
  // below F) and forms the du half of the same columns in the same tile
  const int64_t n_ct = ((SRC == kSrcSwigluBwd ? sw.F : cols) + TC - 1) / TC;
  const int n_rt = gr.tile0[gr.n];
  const int total = (int)((int64_t)((n_rt + 1) / 2) * 2 * n_ct);
  const int id = xcd_remap<kFp4CastChunk>((int)blockIdx.x, total);
  const int64_t pair = id / (2 * n_ct), rem = id - pair * 2 * n_ct;
  const int rt = (int)(2 * pair + (rem & 1));
  if (rt >= n_rt) return;                    // the missing half of an odd last pair
  const int64_t c0 = (rem >> 1) * TC;
  int lo = 0, hi = gr.n - 1;                 // last group whose first tile is <= rt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gr.tile0[mid] <= rt) lo = mid; else hi = mid - 1;
  }
  const int64_t lr0 = (int64_t)(rt - gr.tile0[lo]) * TR;   // first row of the tile in its group
  const int64_t r0 = gr.row0[lo] + lr0;                     // its global row
  const int64_t m_g = gr.row0[lo + 1] - gr.row0[lo];
  const int64_t p_g = (m_g + 31) / 32 * 32;
  const int tid = threadIdx.x;
  const int cc = tid & 15;
  const int64_t col = c0 + cc * VPT;
  const bool col_ok = col < cols;              // cols % 32 == 0: a chunk is wholly in or out

  uint4 raw[TR / 16];
  uint4 raw_u[SRC == kSrcSwigluBwd ? TR / 16 : 1];   // the backward's du values
  if constexpr (SRC == kSrcX) {
    // unconditional loads from clamped addresses (the tile's first row and
    // column), all issued, then zeroed where out of range: a load under the
    // condition is waited for at the branch join, one latency after another
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      const bool ok = lr0 + rr < m_g && col_ok;
      raw[p] = *reinterpret_cast<const uint4*>(x + (r0 + (ok ? rr : 0)) * cols + (ok ? col : c0));
    }
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      if (!(lr0 + rr < m_g && col_ok)) raw[p] = make_uint4(0, 0, 0, 0);
    }
  } else if constexpr (SRC == kSrcSwigluFwd) {
    // A = w * silu(g) * u of 4 columns per row piece, g and u from H1 (fp32)
    static_assert(sizeof(T) == 4, "the SwiGLU sources are fp32");
    const int64_t F = sw.F;
    float4 gv[TR / 16], uv[TR / 16];
    float wv[TR / 16];
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      // routing weight, loaded unconditionally (row clamped; without probs
      // the unit weight kUnitWeight)
      wv[p] = *(sw.probs != nullptr ? sw.probs + r0 + (lr0 + rr < m_g ? rr : 0) : &kUnitWeight);
    }
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      const bool ok = lr0 + rr < m_g && col_ok;
      const float* hp = sw.h1f + (r0 + (ok ? rr : 0)) * 2 * F + (ok ? col : c0);   // clamped, loaded unconditionally
      gv[p] = *reinterpret_cast<const float4*>(hp);
      uv[p] = *reinterpret_cast<const float4*>(hp + F);
    }
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      if (!(lr0 + rr < m_g && col_ok)) {
        gv[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        uv[p] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      const bool ok = lr0 + rr < m_g && col_ok;
      const float w = ok ? wv[p] : 1.0f;
      const float g[4] = {gv[p].x, gv[p].y, gv[p].z, gv[p].w}, u[4] = {uv[p].x, uv[p].y, uv[p].z, uv[p].w};
      uint32_t ab[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g[i]));
        ab[i] = __float_as_uint(w * (g[i] * sig) * u[i]);
      }
      raw[p] = make_uint4(ab[0], ab[1], ab[2], ab[3]);
      if (ok && sw.h1_out != nullptr) {
        uint16_t* hp = sw.h1_out + (r0 + rr) * 2 * F + col;
        *reinterpret_cast<uint2*>(hp) = make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
        *reinterpret_cast<uint2*>(hp + F) = make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
      }
    }
  } else {
    // dg = dA w u s (1 + g (1 - s)) (columns below F) or du = dA w silu(g)
    // (columns F + j), s = sigmoid(g), g and u from the saved bf16 H1; the
    // dg tiles also sum dA silu(g) u over the tile's 64 columns of each row
    static_assert(sizeof(T) == 4, "the SwiGLU sources are fp32");
    const int64_t F = sw.F;
    const int64_t j = col;                      // c0 < F: the tile's columns of dA, g and u
    float4 dv[TR / 16];
    uint2 gq[TR / 16], uq[TR / 16];
    float wv[TR / 16];
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      // loaded unconditionally from clamped addresses (the tile's first row
      // and column), zeroed after
      const int rr = 16 * p + (tid >> 4);
      const bool ok = lr0 + rr < m_g && col_ok;
      const int64_t rc = r0 + (ok ? rr : 0), jc = ok ? j : c0;
      const float4 dl = *reinterpret_cast<const float4*>(sw.da + rc * F + jc);
      const uint16_t* hp = sw.h1 + rc * 2 * F + jc;
      const uint2 gl = *reinterpret_cast<const uint2*>(hp), ul = *reinterpret_cast<const uint2*>(hp + F);
      wv[p] = *(sw.probs != nullptr ? sw.probs + rc : &kUnitWeight);
      dv[p] = ok ? dl : make_float4(0.f, 0.f, 0.f, 0.f);
      gq[p] = ok ? gl : make_uint2(0, 0);
      uq[p] = ok ? ul : make_uint2(0, 0);
    }
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      const bool ok = lr0 + rr < m_g && col_ok;
      const float w = ok ? wv[p] : 1.0f;
      const float d[4] = {dv[p].x, dv[p].y, dv[p].z, dv[p].w};
      const float g[4] = {bf16_lo(gq[p].x), bf16_hi(gq[p].x), bf16_lo(gq[p].y), bf16_hi(gq[p].y)};
      const float u[4] = {bf16_lo(uq[p].x), bf16_hi(uq[p].x), bf16_lo(uq[p].y), bf16_hi(uq[p].y)};
      uint32_t vb[4], vu[4];
      float dp = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[i]));
        const float sl = g[i] * sg;
        vb[i] = __float_as_uint(d[i] * w * u[i] * sg * (1.0f + g[i] * (1.0f - sg)));
        vu[i] = __float_as_uint(d[i] * w * sl);
        dp += d[i] * sl * u[i];
      }
      raw[p] = make_uint4(vb[0], vb[1], vb[2], vb[3]);
      raw_u[p] = make_uint4(vu[0], vu[1], vu[2], vu[3]);
      // the row's 16 chunks of this tile (lanes with the same tid / 16)
#pragma unroll
      for (int sh = 1; sh < 16; sh <<= 1) dp += xor_f32(dp, sh);
      if (cc == 0 && ok && sw.dprobs_part != nullptr) sw.dprobs_part[(c0 / TC) * sw.R + r0 + rr] = dp;
    }
  }
  // every load above is issued before the stores below start (the scheduler
  // would otherwise pair each load with its LDS store and wait in between)
  __builtin_amdgcn_sched_barrier(0);
  // Both layouts of one tile of values (vals) at output columns c0e ..
  // c0e + TC - 1: rowwise codes from registers, then the tile through LDS for
  // the columnwise codes and scales.
  auto emit = [&](const uint4 (&vals)[TR / 16], int64_t c0e) __attribute__((always_inline)) {
    const int64_t c0 = c0e;
    const int64_t col = c0 + cc * VPT;
    const bool col_ok = col < cols;
  #pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int rr = 16 * p + (tid >> 4);
      *reinterpret_cast<uint4*>(tile + rr * 256 + cc * 16) = vals[p];
      if (q_row != nullptr) {
        float v[VPT];
        if constexpr (kBf16) {
          v[0] = bf16_lo(vals[p].x); v[1] = bf16_hi(vals[p].x); v[2] = bf16_lo(vals[p].y); v[3] = bf16_hi(vals[p].y);
          v[4] = bf16_lo(vals[p].z); v[5] = bf16_hi(vals[p].z); v[6] = bf16_lo(vals[p].w); v[7] = bf16_hi(vals[p].w);
        } else {
          v[0] = __uint_as_float(vals[p].x); v[1] = __uint_as_float(vals[p].y);
          v[2] = __uint_as_float(vals[p].z); v[3] = __uint_as_float(vals[p].w);
        }
        uint32_t am = 0;
  #pragma unroll
        for (int i = 0; i < VPT; ++i) am = umax(am, abs_bits(v[i]));
  #pragma unroll
        for (int sh = 1; sh < TPB; sh <<= 1) am = umax(am, xor_u32(am, sh));
        const uint32_t eb = am >> 23;
        const uint32_t sc = eb > 2u ? eb - 2u : 0u;
        uint32_t codes;
        if constexpr (kBf16) {
          codes = e2m1x8_bf16(vals[p], e8m0_as_scale(sc));
        } else {
          codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], e8m0_as_scale(sc), 0);
          codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, v[2], v[3], e8m0_as_scale(sc), 1);
        }
        const int64_t row = r0 + rr;
        const bool row_ok = lr0 + rr < m_g;
        if (row_ok && col_ok) {
          if constexpr (kBf16) *reinterpret_cast<uint32_t*>(q_row + row * (cols / 2) + col / 2) = codes;
          else *reinterpret_cast<uint16_t*>(q_row + row * (cols / 2) + col / 2) = (uint16_t)codes;
        }
        // the row's scale bytes of this tile, gathered into one word
        uint32_t word = sc << (8 * (cc / TPB));
  #pragma unroll
        for (int sh = TPB; sh < 16; sh <<= 1) word |= xor_u32(word, sh);
        if (cc == 0 && row_ok) {
          uint8_t* sd = s_row + row * (cols / 32) + c0 / 32;
          const bool whole = c0 + TC <= cols && (reinterpret_cast<uintptr_t>(sd) & (NB - 1)) == 0;
          if (whole) {
            if constexpr (NB == 4) *reinterpret_cast<uint32_t*>(sd) = word;
            else *reinterpret_cast<uint16_t*>(sd) = (uint16_t)word;
          } else {
  #pragma unroll
            for (int j = 0; j < NB; ++j)
              if (c0 + 32 * j < cols) sd[j] = (uint8_t)(word >> (8 * j));
          }
        }
      }
    }
    __syncthreads();

    // columnwise: thread t takes the CPS columns of dword t % 64 and the 32-row
    // block t / 64 (rows of the group past its end are zeros)
    const int rb = tid >> 6, slot = tid & 63;
    float v[CPS][32];
  #pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (32 * rb + i) * 256 + slot * 4);
      if constexpr (kBf16) {
        v[0][i] = bf16_lo(w);
        v[CPS - 1][i] = bf16_hi(w);
      } else {
        v[0][i] = __uint_as_float(w);
      }
    }
    __syncthreads();                             // every column read: the tile becomes the code staging
  #pragma unroll
    for (int j = 0; j < CPS; ++j) {
      uint4 codes;
      const uint32_t sc = fp4_block(v[j], codes);
      const int cl = CPS * slot + j;             // column inside the tile
      *reinterpret_cast<uint4*>(tile + cl * 64 + ((rb ^ ((cl >> 2) & 3)) << 4)) = codes;
      reinterpret_cast<uint8_t*>(cs_t)[cl * 4 + rb] = (uint8_t)sc;
    }
    __syncthreads();

    // each column's 64-byte run; blocks past the group's padded rows are not
    // part of the layout (the next group's columns start there)
    const int64_t pc0 = gr.pcol0[lo] + lr0;     // the tile's first position in the columnwise layout
  #pragma unroll
    for (int it = 0; it < TC * 4 / 256; ++it) {
      const int u = it * 256 + tid;
      const int cl = u >> 2, piece = u & 3;
      const int64_t colc = c0 + cl;
      if (colc < cols && lr0 + 32 * piece < p_g)
        *reinterpret_cast<uint4*>(q + colc * (ldp / 2) + pc0 / 2 + 16 * piece) =
            *reinterpret_cast<const uint4*>(tile + cl * 64 + ((piece ^ ((cl >> 2) & 3)) << 4));
    }
    // columnwise scales: the tile's 4 blocks of a column are 4 consecutive bytes
    if (tid < TC) {
      const int64_t colc = c0 + tid;
      if (colc < cols) {
        const uint32_t word = cs_t[tid];
        uint8_t* sd = s + colc * (ldp / 32) + pc0 / 32;
        if (lr0 + 96 < p_g && (reinterpret_cast<uintptr_t>(sd) & 3) == 0) {
          *reinterpret_cast<uint32_t*>(sd) = word;
        } else {
  #pragma unroll
          for (int j = 0; j < 4; ++j)
            if (lr0 + 32 * j < p_g) sd[j] = (uint8_t)(word >> (8 * j));
        }
      }
    }
  };
  emit(raw, c0);
  if constexpr (SRC == kSrcSwigluBwd) {
    __syncthreads();                           // the LDS tile and scale words are free again
    emit(raw_u, sw.F + c0);
  }
}

// Grid of the columnwise cast: row tiles in pairs, times the column tiles.
template <typename T>
int64_t fp4_colwise_grid(const Fp4ColGroups& gr, int64_t cols) {
  constexpr int TC = 16 * (16 / (int)sizeof(T));
  return (int64_t)((gr.tile0[gr.n] + 1) / 2) * 2 * ((cols + TC - 1) / TC);
}

hipError_t launch_quantize_fp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                               uint8_t* s_col, hipStream_t stream) {
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  // both layouts: one pass (the columnwise kernel writes the rowwise pair too)
  const bool fused = q != nullptr && q_col != nullptr;
  const int64_t blocks = q != nullptr && !fused ? rows * (cols / 32) : 0;
  if (blocks > 0)
    hipLaunchKernelGGL(quantize_fp4_rowwise_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream,
                       xb, rows, cols, q, s);
  if (q_col != nullptr && rows > 0) {
    Fp4ColGroups gr{};
    gr.n = 1;
    gr.row0[0] = 0;
    gr.row0[1] = rows;
    gr.pcol0[0] = 0;
    gr.pcol0[1] = rows;
    gr.tile0[0] = 0;
    gr.tile0[1] = (int32_t)((rows + kFp4ColTileRows - 1) / kFp4ColTileRows);
    const int64_t tiles = fp4_colwise_grid<uint16_t>(gr, cols);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_fp4_colwise_kernel<uint16_t>, dim3((unsigned)tiles), dim3(256), 0, stream, xb, rows,
                       cols, q_col, s_col, fused ? q : nullptr, fused ? s : nullptr, gr, rows, Fp4SwigluArgs{});
  }
  return hipGetLastError();
}

hipError_t launch_quantize_fp4_grouped(const void* x, bool x_f32, int64_t rows, int64_t cols, const Fp4ColGroups& gr,
                                       uint8_t* q_col, uint8_t* s_col, uint8_t* q_row, uint8_t* s_row,
                                       hipStream_t stream) {
  const int64_t tiles = x_f32 ? fp4_colwise_grid<float>(gr, cols) : fp4_colwise_grid<uint16_t>(gr, cols);
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (x_f32)
    hipLaunchKernelGGL(quantize_fp4_colwise_kernel<float>, dim3((unsigned)tiles), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(x), rows, cols, q_col, s_col, q_row, s_row, gr,
                       (int64_t)gr.pcol0[gr.n], Fp4SwigluArgs{});
  else
    hipLaunchKernelGGL(quantize_fp4_colwise_kernel<uint16_t>, dim3((unsigned)tiles), dim3(256), 0, stream,
                       reinterpret_cast<const uint16_t*>(x), rows, cols, q_col, s_col, q_row, s_row, gr,
                       (int64_t)gr.pcol0[gr.n], Fp4SwigluArgs{});
  return hipGetLastError();
}

hipError_t launch_swiglu_fp4_cast(bool backward, const Fp4SwigluArgs& sw, const Fp4ColGroups& gr, uint8_t* q_col,
                                  uint8_t* s_col, uint8_t* q_row, uint8_t* s_row, hipStream_t stream) {
  const int64_t cols = backward ? 2 * sw.F : sw.F;
  if (sw.F % 128 != 0) return hipErrorInvalidValue;
  // the backward's tiles cover the F columns of dA and each writes both dg and du
  const int64_t tiles = fp4_colwise_grid<float>(gr, sw.F);
  if (tiles == 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (backward)
    hipLaunchKernelGGL((quantize_fp4_colwise_kernel<float, kSrcSwigluBwd>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, nullptr, sw.R, cols, q_col, s_col, q_row, s_row, gr, (int64_t)gr.pcol0[gr.n], sw);
  else
    hipLaunchKernelGGL((quantize_fp4_colwise_kernel<float, kSrcSwigluFwd>), dim3((unsigned)tiles), dim3(256), 0,
                       stream, nullptr, sw.R, cols, q_col, s_col, q_row, s_row, gr, (int64_t)gr.pcol0[gr.n], sw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// NVFP4: E2M1 elements in blocks of 16 values, one E4M3 scale per block and
// one fp32 scale per tensor (the NVFP4 recipe of "TransformerEngine-
// accelerated Llama 3 training with native PyTorch training loop", Quantized
// Training; the format's published form). With the tensor's amax, in fp32
// arithmetic rounded to nearest:
//   S   = 2688 / amax (448 * 6), 1 for amax = 0, at most 2^64;
//   s_b = E4M3 code of (bmax / 6) * S, saturating;
//   q   = E2M1 code of x * (S / E4M3(s_b)) (0, keeping the sign, when s_b = 0).
// An element's value is E2M1(q) * E4M3(s_b) / S.

__device__ __forceinline__ float nvfp4_tensor_scale(float amax) {
  if (!(amax > 0.0f)) return 1.0f;
  return fminf(2688.0f / amax, 18446744073709551616.0f);   // cap 2^64
}

// 16 values -> 8 code bytes (element 2i in the low nibble) and the E4M3
// block-scale code.
__device__ __forceinline__ uint32_t nvfp4_block(const float (&v)[16], float S, uint2& codes) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = umax(am, abs_bits(v[i]));
  const float t = __uint_as_float(am) / 6.0f;
  const float sb = t * S;
  const uint32_t sc = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(sb, 448.0f), 0.0f, 0, false) & 0xFFu;
  const float sv = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
  const float r = sv > 0.0f ? S / sv : 0.0f;
  // q = E2M1 of fl32(v * r): the convert at scale 1 (E8M0 code 127)
  float vr[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) vr[j] = v[j] * r;
  codes = make_uint2(e2m1x8(&vr[0], 1.0f), e2m1x8(&vr[8], 1.0f));
  return sc;
}

__global__ void nvfp4_amax_init_kernel(uint32_t* amax_bits) { *amax_bits = 0u; }

// max |x| over the tensor: per-thread maxima of the magnitude bits (bf16 bits
// shifted into fp32 position order the same way as the values), wave and
// workgroup maxima, one atomic maximum per workgroup.
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const uint16_t* x, int64_t n8, uint32_t* amax_bits) {
  uint32_t m = 0;
  const uint4* src = reinterpret_cast<const uint4*>(x);
  auto take = [&](const uint4& v) __attribute__((always_inline)) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = umax(m, (w[j] << 16) & 0x7FFFFFFFu);
      m = umax(m, w[j] & 0x7FFF0000u);
    }
  };
  // four independent 16-byte loads in flight per thread, then the remainder
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
    take(v0);
    take(v1);
    take(v2);
    take(v3);
  }
  for (; i < n8; i += stride) take(src[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  // one atomic per workgroup: atomics on one address serialize
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(amax_bits, umax(umax(wmax[0], wmax[1]), umax(wmax[2], wmax[3])));
}

// Rowwise and/or columnwise NVFP4 of bf16 x [rows, cols] from one LDS tile of
// 128 rows x 64 columns: the rowwise copy takes 16-column blocks of each
// row, the columnwise copy 16-row blocks of each column (the rowwise copy of
// the transpose); both use the tensor scale of amax.
constexpr int kNvTileRows = 128, kNvTileCols = 64;
__global__ __launch_bounds__(256) void nvfp4_cast_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                         const float* amax, uint8_t* q, uint8_t* s, uint8_t* qc,
                                                         uint8_t* sc) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kNvTileRows][kNvTileCols + 2];
  const int64_t n_ct = (cols + kNvTileCols - 1) / kNvTileCols;
  const int64_t r0 = (int64_t)(blockIdx.x / n_ct) * kNvTileRows, c0 = (int64_t)(blockIdx.x % n_ct) * kNvTileCols;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int p = it * 256 + tid, rr = p >> 3, cp = (p & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < rows && c0 + cp < cols) v = *reinterpret_cast<const uint4*>(x + (r0 + rr) * cols + c0 + cp);
    const uint16_t e[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                           (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][cp + j] = e[j];
  }
  __syncthreads();
  const float S = nvfp4_tensor_scale(*amax);
  if (q != nullptr) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int task = tid + 256 * u, rr = task >> 2, blk = task & 3;
      const int64_t row = r0 + rr, col = c0 + 16 * blk;
      if (row < rows && col < cols) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __uint_as_float((uint32_t)tile[rr][16 * blk + i] << 16);
        uint2 codes;
        const uint32_t code = nvfp4_block(v, S, codes);
        *reinterpret_cast<uint2*>(q + row * (cols / 2) + col / 2) = codes;
        s[row * (cols / 16) + col / 16] = (uint8_t)code;
      }
    }
  }
  if (qc != nullptr) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int task = tid + 256 * u, cc = task & 63, rb = task >> 6;
      const int64_t col = c0 + cc, row = r0 + 16 * rb;
      if (col < cols && row < rows) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __uint_as_float((uint32_t)tile[16 * rb + i][cc] << 16);
        uint2 codes;
        const uint32_t code = nvfp4_block(v, S, codes);
        *reinterpret_cast<uint2*>(qc + col * (rows / 2) + row / 2) = codes;
        sc[col * (rows / 16) + row / 16] = (uint8_t)code;
      }
    }
  }
}

hipError_t launch_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                                 uint8_t* s_col, float* amax, hipStream_t stream) {
  uint32_t* ab = reinterpret_cast<uint32_t*>(amax);
  hipLaunchKernelGGL(nvfp4_amax_init_kernel, dim3(1), dim3(1), 0, stream, ab);
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipGetLastError();
  const int64_t grid = std::min<int64_t>((n8 + 255) / 256, 512);
  hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), n8, ab);
  const int64_t tiles = ((rows + kNvTileRows - 1) / kNvTileRows) * ((cols + kNvTileCols - 1) / kNvTileCols);
  hipLaunchKernelGGL(nvfp4_cast_kernel, dim3((unsigned)tiles), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(x), rows, cols, amax, q, s, q_col, s_col);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// ScaledSwiGLU around the MXFP4 GEMMs of the MLP ("Efficient MoE training for
// biological foundation models", Key technical approaches item 3, at the 4-bit
// MX format): GEMM1 leaves H1 = [g | u] in fp32 and dgrad2 leaves dA in fp32.
// In training the columnwise cast forms A = w * silu(g) * u, resp.
// dH1 = [dg | du] and dprobs, on the fly (launch_swiglu_fp4_cast); silu and
// its derivative use the same fp32 expressions as the MXFP8 epilogues.

// Inference forward: one thread per (row, 32-column block of F), A's rowwise
// MXFP4 copy only.
__global__ __launch_bounds__(256) void swiglu_fwd_fp4_kernel(const float* h1f, const float* probs, int64_t R,
                                                             int64_t F, uint8_t* aq, uint8_t* as) {
  const int64_t nb = F / 32;
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= R * nb) return;
  const int64_t r = blk / nb, b = blk - r * nb;
  const float4* gp = reinterpret_cast<const float4*>(h1f + r * 2 * F + 32 * b);
  const float4* up = reinterpret_cast<const float4*>(h1f + r * 2 * F + F + 32 * b);
  float g[32], u[32], a[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 gv = gp[i], uv = up[i];
    g[4 * i] = gv.x; g[4 * i + 1] = gv.y; g[4 * i + 2] = gv.z; g[4 * i + 3] = gv.w;
    u[4 * i] = uv.x; u[4 * i + 1] = uv.y; u[4 * i + 2] = uv.z; u[4 * i + 3] = uv.w;
  }
  const float w = probs != nullptr ? probs[r] : 1.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-g[i]));
    a[i] = w * (g[i] * sig) * u[i];
  }
  uint4 codes;
  const uint32_t sc = fp4_block(a, codes);
  *reinterpret_cast<uint4*>(aq + r * (F / 2) + 16 * b) = codes;
  as[r * nb + b] = (uint8_t)sc;
}

hipError_t launch_swiglu_fwd_fp4(const float* h1f, const float* probs, int64_t R, int64_t F, uint8_t* aq, uint8_t* as,
                                 hipStream_t stream) {
  const int64_t blocks = R * (F / 32);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_fp4_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream, h1f, probs,
                     R, F, aq, as);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP4 grouped GEMM: the rows of A [M, K] are split into groups (per-expert
// split_sizes, GroupedLinear); the rows of group g get C = A_g . B_g^T with
// B_g [N, K] the group's weight. Both operands are in the rowwise MXFP4 layout
// of the cast above (codes [rows, K/2], scales [rows, K/32]). One group is
// the plain GEMM. Runs on gfx950's scaled MFMA with both operand formats set
// to E2M1; every product of two E2M1 values is exact, the instruction
// accumulates in fp32. M-tiles restart at each group's first row.
//
// Workgroup tile 256 x 256: four waves in 2 x 2, each 4 x 4 MFMA tiles of
// 32 x 32 x 64 (128 x 128 fp32 accumulators in AGPRs). Operands are read through buffer resources, so rows past M
// or N read as zeros. E2M1 operand layout (pinned on
// hardware): lane l holds row l % 32 and, with h = l / 32, the 32 values
// k [32h, 32h+32) of the k-step in the 16 bytes of its first four operand
// registers, in memory order; its scale register scales that block. (The FP8
// operand splits each lane's 32 values into two 16-value halves instead.)

// A k-tile is 256 values (128 bytes of codes) of every row of the workgroup
// tile; A and B k-tiles are staged in LDS, double-buffered, by buffer->LDS DMA
// (8 lanes per 128-byte row), with 16-byte chunk c of row r at chunk
// c ^ ((r >> 1) & 7): two 128-byte rows share one 256-byte line of the 64 LDS
// banks, so this puts a fragment read's 16 consecutive rows (one chunk each)
// on 16 different 16-byte bank groups. One barrier per k-tile: the next k-tile's DMA is in flight during
// this one's MFMAs.
constexpr int kF4SubM = 4, kF4SubN = 4;     // wave tile: MFMA tiles of 32 x 32
constexpr int kF4BandM = 4;                 // group-K: m-tiles per band of the tile raster
constexpr int kF4KTile = 128;               // bytes of codes per row and k-tile
static_assert(kFp4GemmTileM == 2 * 32 * kF4SubM && kFp4GemmTileN == 2 * 32 * kF4SubN, "tile = 2 x 2 waves");

// GK: the group-K (weight-gradient) form. The workgroup takes tile (mt, nt)
// of group g's output C_g [M, N] (all groups' tiles in group order), over
// group g's k range [k0[g], k0[g+1]) of A [M, K] and B [N, K]; a last k-step
// that holds only 32 valid values gets scale code 0 for the invalid half on
// both operands, so its products (at most 36 * 2^-254) add exact zeros
// whatever codes lie past the group; C_g is fp32, stored or accumulated.
// SPLIT: the split-K tail units only (a launch of its own over
// (tiles - sp.first) * sp.parts workgroups), fp32 partial tiles out.
template <bool GK, bool F32, bool NV, bool SPLIT = false>
__global__ __launch_bounds__(256) void gemm_fp4_kernel(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                                       const uint8_t* bs, Fp4Groups gr, Fp4KGroups kg, int64_t M,
                                                       int64_t N, int64_t K, int64_t n_tiles_n, void* c,
                                                       int32_t accumulate,
                                                       const float* a_amax, const float* b_amax, Fp4Split sp) {
  constexpr int SM = kF4SubM, SN = kF4SubN, TM = kFp4GemmTileM, TN = kFp4GemmTileN, KT = kF4KTile;
  constexpr uint32_t kE2M1 = 4;               // operand format selector of the scaled MFMA
  // The two stages of A and B as four separate LDS objects, the stage of each
  // k-tile fixed at compile time (the k-loop is unrolled by two): the
  // compiler then sees that the DMA into one stage never aliases the
  // fragment reads of the other and does not wait for the next k-tile's
  // loads before computing on this one.
  __shared__ __attribute__((aligned(16))) uint8_t sA0[TM * KT];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[TM * KT];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[TN * KT];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[TN * KT];
  static_assert(TM * KT == 2 * SN * 4096 && TN * KT == 2 * SN * 4096,
                "each wave's fp32 epilogue slice is one whole stage array");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;
  int grp;   // the group (expert) of this tile
  int64_t row_end, am0, bn0, kbeg = 0, klen = K;
  // Tile id. Group-K: consecutive ids (raster neighbours) run together on one
  // XCD. Group-M keeps the launch order: with a multiple of 8 n-tiles, block
  // b's n-tile (and its rows of B) stays on XCD b % 8 for every m-tile.
  const int64_t per_group = GK ? ((M + TM - 1) / TM) * n_tiles_n : 0;
  int id = GK ? xcd_remap((int)blockIdx.x, (int)(kg.n * per_group)) : (int)blockIdx.x;
  // split-K tail units: workgroup u is part u % parts of tile first + u / parts
  int split_unit = -1, part = 0;
  if constexpr (SPLIT) {
    split_unit = (int)blockIdx.x;
    id = sp.first + split_unit / sp.parts;
    part = split_unit % sp.parts;
  }
  if constexpr (GK) {
    // Every group has per_group tiles. When that is a multiple of kXcdChunk,
    // chunk q of kXcdChunk ids goes to group (q % n + q / n) % n as its chunk
    // q / n: the tiles running at one time mix groups of different k lengths
    // (k-loops and fp32 stores overlap across CUs) while one XCD's chunk
    // stays inside one group.
    int64_t rem;
    if (per_group % kXcdChunk == 0) {
      const int64_t q = id / kXcdChunk, r = q / kg.n, pos = q - r * kg.n;
      grp = (int)((pos + r) % kg.n);
      rem = r * kXcdChunk + (id - q * kXcdChunk);
    } else {
      grp = (int)(id / per_group);
      rem = id - grp * per_group;
    }
    // bands of kF4BandM m-tiles x all n-tiles, m fastest inside a band: a
    // chunk of 32 ids is 4 m-tiles x 8 n-tiles, which share their A and B
    // rows in the XCD's L2
    const int64_t m_tiles = (M + TM - 1) / TM, per_band = kF4BandM * n_tiles_n;
    const int64_t band = rem / per_band, in_band = rem - band * per_band;
    const int64_t band_h = min<int64_t>(kF4BandM, m_tiles - band * kF4BandM);
    const int64_t mt = band * kF4BandM + in_band % band_h, nt = in_band / band_h;
    row_end = M;
    am0 = mt * TM;
    bn0 = nt * TN;
    kbeg = kg.k0[grp];
    klen = kg.k0[grp + 1] - kbeg;
  } else {
    const int64_t mt = id / n_tiles_n, nt = id - mt * n_tiles_n;
    // group of m-tile mt: the last group whose first m-tile is <= mt (empty
    // groups own no m-tile)
    int lo = 0, hi = gr.n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gr.tile0[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    grp = lo;
    row_end = gr.row0[grp + 1];               // rows of the group end here
    am0 = gr.row0[grp] + (mt - gr.tile0[grp]) * TM;
    bn0 = nt * TN;
  }
  const int64_t amv = min<int64_t>(TM, row_end - am0), bnv = min<int64_t>(TN, N - bn0);
  // bytes per row of codes, of scales (one per 32 values; NVFP4: per 16)
  constexpr int kVPS = NV ? 16 : 32;           // values per scale
  const int64_t ldq = K / 2, lds = K / kVPS;
  // group-M: B_g is rows [g N, g N + N) of b; group-K: one B, the group's k range
  const int64_t brow0 = GK ? bn0 : grp * N + bn0;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a + am0 * ldq + kbeg / 2, (amv - 1) * ldq + klen / 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(b + brow0 * ldq + kbeg / 2, (bnv - 1) * ldq + klen / 2);
  // a row's 8 scales of a k-tile: one aligned 8-byte load (sc_dword). The k
  // range must also be whole k-tiles: the last row's load would otherwise
  // reach past the resource's extent and come back as zero scales. (NVFP4: K
  // is a multiple of 128, so a lane's 8 scales of a k-tile are always one
  // aligned 8-byte piece.) Group-K ranges start at any multiple of 32 values,
  // so a group's scales start at any byte: group-K takes (sc_shift) the
  // aligned 16 bytes around the 8 and a per-lane byte shift (0 where they are
  // aligned), through resources over the whole scale arrays (offsets from
  // their bases, which the range check covers). A load that reaches past the
  // extent reads zeros, also for its bytes inside it, so a lane whose 16
  // bytes do not all lie in the array (the array's last row or two) takes
  // byte loads. One load shape for all group-K tiles also keeps the combine
  // from waiting (an 8-byte path beside it made the compiler copy its
  // result, which waits for the load). Else byte loads throughout.
  const bool sc_dword = NV || ((lds & 7) == 0 && ((kbeg / 32) & 7) == 0 && ((klen / 32) & 7) == 0);
  const bool sc_shift = GK &&
                        ((reinterpret_cast<uintptr_t>(as) | reinterpret_cast<uintptr_t>(bs)) & 7) == 0 &&
                        M * lds < ((int64_t)1 << 32) && N * lds < ((int64_t)1 << 32);
  const int64_t sa_len = sc_shift ? M * lds : (amv - 1) * lds + klen / kVPS;
  const int64_t sb_len = sc_shift ? N * lds : (bnv - 1) * lds + klen / kVPS;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sc_shift ? as : as + am0 * lds + kbeg / kVPS, sa_len);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(sc_shift ? bs : bs + brow0 * lds + kbeg / kVPS, sb_len);
  const uint32_t sa_off0 = sc_shift ? (uint32_t)(am0 * lds + kbeg / 32) : 0u;
  const uint32_t sb_off0 = sc_shift ? (uint32_t)(brow0 * lds + kbeg / 32) : 0u;
  const int ksteps = (int)((klen + 63) / 64), ktiles = (ksteps + 3) / 4;
  // k-tiles [t_lo, t_hi) of this work unit
  const int t_lo = SPLIT ? part * ktiles / sp.parts : 0;
  const int t_hi = SPLIT ? (part + 1) * ktiles / sp.parts : ktiles;

  // global -> LDS by buffer DMA, 1 KB (8 rows) per instruction: lane L
  // fills chunk L % 8 of row 8 blk + L / 8 with global chunk
  // (L % 8) ^ (((8 blk + L / 8) >> 1) & 7) = (L % 8) ^ (L / 16) ^ 4 (blk & 1),
  // the swizzle above; blk = 4 p + wave, so blk & 1 = wave & 1. Bytes past K
  // in the last k-tile come from the next row (or read zero) and feed only
  // skipped k-steps.
  const uint32_t dma_off = (uint32_t)((lane >> 3) * ldq + 16 * ((lane & 7) ^ (lane >> 4) ^ (4 * (wave & 1))));
  auto dma_tile = [&](int t, uint8_t* dA, uint8_t* dB) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < TM / 32; ++p) {
      const int blk = 4 * p + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dA + blk * 1024), 16, dma_off,
                                               (uint32_t)(8 * blk * ldq + KT * t), 0, 0);
    }
#pragma unroll
    for (int p = 0; p < TN / 32; ++p) {
      const int blk = 4 * p + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dB + blk * 1024), 16, dma_off,
                                               (uint32_t)(8 * blk * ldq + KT * t), 0, 0);
    }
  };
  // scales of k-tile t for this lane's rows: blocks 8 t .. 8 t + 7 (NVFP4:
  // blocks 16 t + 8 h .. + 7, those of the lane's half of the k-tile)
  u32x2 sca[SM], scb[SN];
  const uint32_t sc_k = NV ? 8 * h : 0;
  // A lane's scales of one k-tile in two steps: the loads (scale_load, raw
  // words: the 8 scale bytes in x, y, or for sc_shift the two aligned pieces
  // in x, y and z, w), and after the k-tile's wait the byte shift
  // (scale_take), so that combining the pieces never waits on the loads
  // issued with them, the next k-tile's DMA among them.
  auto shifted = [&](uint32_t off, int64_t len) __attribute__((always_inline)) -> bool {
    return sc_shift && (int64_t)(off & ~7u) + 16 <= len;
  };
  auto scale_load = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off, int64_t len)
      __attribute__((always_inline)) -> u32x4 {
    u32x4 w;
    w.z = 0; w.w = 0;
    if (shifted(off, len)) {
      const uint32_t al = off & ~7u;
      const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(r, al, 0, 0);
      const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(r, al + 8, 0, 0);
      w.x = lo.x; w.y = lo.y; w.z = hi.x; w.w = hi.y;
      return w;
    }
    if (sc_dword) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      w.x = v.x; w.y = v.y;
      return w;
    }
    w.x = 0; w.y = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(r, off + e, 0, 0);
      if (e < 4) w.x |= byte << (8 * e); else w.y |= byte << (8 * (e - 4));
    }
    return w;
  };
  auto scale_take = [&](const u32x4& w, uint32_t off, int64_t len) __attribute__((always_inline)) -> u32x2 {
    u32x2 v;
    if (shifted(off, len)) {
      const uint32_t sh = off & 7u;
      const bool up = sh >= 4;                // the 8 bytes start in the second dword
      const uint32_t a0 = up ? w.y : w.x, a1 = up ? w.z : w.y, a2 = up ? w.w : w.z;
      v.x = __builtin_amdgcn_alignbyte(a1, a0, sh & 3u);
      v.y = __builtin_amdgcn_alignbyte(a2, a1, sh & 3u);
    } else {
      v.x = w.x; v.y = w.y;
    }
    return v;
  };
  auto sa_off = [&](int t, int i) __attribute__((always_inline)) -> uint32_t {
    return sa_off0 + (uint32_t)((TM / 2 * wm + 32 * i + l32) * lds + (NV ? 16 : 8) * t + sc_k);
  };
  auto sb_off = [&](int t, int j) __attribute__((always_inline)) -> uint32_t {
    return sb_off0 + (uint32_t)((TN / 2 * wn + 32 * j + l32) * lds + (NV ? 16 : 8) * t + sc_k);
  };
  auto load_scales = [&](int t, u32x4 (&xa)[SM], u32x4 (&xb)[SN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SM; ++i) xa[i] = scale_load(rsa, sa_off(t, i), sa_len);
#pragma unroll
    for (int j = 0; j < SN; ++j) xb[j] = scale_load(rsb, sb_off(t, j), sb_len);
  };
  auto take_scales = [&](int t, const u32x4 (&xa)[SM], const u32x4 (&xb)[SN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SM; ++i) sca[i] = scale_take(xa[i], sa_off(t, i), sa_len);
#pragma unroll
    for (int j = 0; j < SN; ++j) scb[j] = scale_take(xb[j], sb_off(t, j), sb_len);
  };
  auto frag = [&](const uint8_t* base, int r, int s) __attribute__((always_inline)) -> v8i {
    const u32x4 q = *reinterpret_cast<const u32x4*>(base + r * KT + (((2 * s + h) ^ ((r >> 1) & 7)) << 4));
    v8i f;
    f[0] = q.x; f[1] = q.y; f[2] = q.z; f[3] = q.w;
    f[4] = 0; f[5] = 0; f[6] = 0; f[7] = 0;
    return f;
  };
  auto pick = [&](const u32x2& v, int s) __attribute__((always_inline)) -> int {
    const int blk = 2 * s + h;               // this lane's block of k-step s
    return (int)(((blk < 4 ? v.x : v.y) >> (8 * (blk & 3))) & 0xFFu);
  };

  v16f acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[j][i][v] = 0.0f;

  // L2 prefetch (MXFP4): once the loads of k-tile t + 1 are out, each wave
  // touches one 128-byte line in each of 128 rows of k-tile t + kF4Prefetch
  // (waves 0-1 the tile's A rows, waves 2-3 its B rows), so that k-tile's
  // DMA finds its lines in L2. The two words land in a register pair of the
  // k-tile's parity (the loop is unrolled by two, so the pairs alternate
  // without moves); the wait at the end of the k-tile leaves them in flight,
  // and at the end of the next k-tile, when in-order completion has them in,
  // they are folded into a sink, so the prefetch adds no wait. (A
  // buffer->LDS touch would not do: the barrier's release fence waits for
  // every LDS write.) Rows and columns past the resource extents read
  // nothing.
  constexpr int kF4Prefetch = 3;
  constexpr int kWaitVmcnt2 = 0x0F72;         // s_waitcnt vmcnt(2), expcnt/lgkmcnt open
  const __amdgpu_buffer_rsrc_t rpf = make_rsrc(wave < 2 ? a + am0 * ldq + kbeg / 2 : b + brow0 * ldq + kbeg / 2,
                                               wave < 2 ? (amv - 1) * ldq + klen / 2 : (bnv - 1) * ldq + klen / 2);
  const uint32_t pf_off = (uint32_t)((128 * (wave & 1) + lane) * ldq);
  uint32_t pf_sink = 0, pf_even[2] = {0u, 0u}, pf_odd[2] = {0u, 0u};
  auto prefetch = [&](int t, uint32_t (&d)[2]) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)(KT * t);
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(rpf, pf_off, k0, 0);
    d[1] = __builtin_amdgcn_raw_buffer_load_b32(rpf, pf_off + (uint32_t)(64 * ldq), k0, 0);
  };

  u32x4 nsa[SM], nsb[SN];
  dma_tile(t_lo, sA0, sB0);
  load_scales(t_lo, nsa, nsb);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  take_scales(t_lo, nsa, nsb);
  __syncthreads();
  // k-tile t on stage (cA, cB) while k-tile t + 1 loads into (nA, nB)
  auto ktile = [&](int t, const uint8_t* cA, const uint8_t* cB, uint8_t* nA, uint8_t* nB, uint32_t (&pf_mine)[2],
                   const uint32_t (&pf_prev)[2]) __attribute__((always_inline)) {
    const bool more = t + 1 < t_hi;           // uniform over the workgroup
    if (more) {
      dma_tile(t + 1, nA, nB);
      load_scales(t + 1, nsa, nsb);
    }
    // unconditional, so that it is the newest load on every path
    if constexpr (!NV) prefetch(t + kF4Prefetch, pf_mine);
    const uint8_t* A = cA + (TM / 2 * wm) * KT;
    const uint8_t* B = cB + (TN / 2 * wn) * KT;
    if constexpr (NV) {
      // NVFP4 on the fp16 MFMA (32 x 32 x 16): the lanes of half h take the
      // values [128 h, 128 h + 128) of the k-tile, read as chunks 4 h .. 4 h + 3
      // of their rows, so step 4 q + u pairs values 32 q + 8 u .. + 7 (h = 0)
      // with 128 + 32 q + 8 u .. + 7 (h = 1) -- the same permutation of k for
      // A and B, and each lane's 8 values lie in one 16-value block. Each
      // lane dequantizes its 8 values exactly into fp16 (E2M1 times an E4M3
      // scale has at most 6 significant bits). A half past K (K % 256 == 128
      // in the last k-tile) gets scale 0.
      const bool half_ok = (int64_t)(256 * t + 128 * h) < klen;
      auto chunk = [&](const uint8_t* base, int r, int c) __attribute__((always_inline)) -> u32x4 {
        return *reinterpret_cast<const u32x4*>(base + r * KT + ((c ^ ((r >> 1) & 7)) << 4));
      };
      auto dequant = [&](uint32_t w, float sv) __attribute__((always_inline)) -> f16x8 {
        // sv = 2^E * m with m in [1, 2) holding at most 3 fraction bits: the
        // scaled conversion applies 2^E exactly, one packed fp16 multiply per
        // pair applies m (exact: at most 6 significant bits, within fp16's
        // normal range 2^-10 .. 2688)
        const uint32_t sb = __float_as_uint(sv);
        const float pe = __uint_as_float(sb & 0x7F800000u);
        const uint32_t mb = 0x3C00u | ((sb >> 13) & 0x3FFu);
        const f16x2 mh = __builtin_bit_cast(f16x2, mb | (mb << 16));
        u32x4 o;
        o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pe, 0) * mh);
        o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pe, 1) * mh);
        o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pe, 2) * mh);
        o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, pe, 3) * mh);
        return __builtin_bit_cast(f16x8, o);
      };
      static_for<0, 4>([&](auto qd_c) __attribute__((always_inline)) {
        constexpr int qd = decltype(qd_c)::value;
        u32x4 cb[SN], ca[SM];
#pragma unroll
        for (int j = 0; j < SN; ++j) cb[j] = chunk(B, 32 * j + l32, qd + 4 * h);
#pragma unroll
        for (int i = 0; i < SM; ++i) ca[i] = chunk(A, 32 * i + l32, qd + 4 * h);
        static_for<0, 4>([&](auto u_c) __attribute__((always_inline)) {
          constexpr int u = decltype(u_c)::value;
          constexpr int blk = 2 * qd + u / 2;             // the lane's block (byte of its scale pair)
          f16x8 fb[SN];
#pragma unroll
          for (int j = 0; j < SN; ++j) {
            const uint32_t sw = blk < 4 ? scb[j].x : scb[j].y;
            const float sv = half_ok ? __builtin_amdgcn_cvt_f32_fp8((int)sw, blk & 3) : 0.0f;
            fb[j] = dequant(cb[j][u], sv);
          }
#pragma unroll
          for (int i = 0; i < SM; ++i) {
            const uint32_t sw = blk < 4 ? sca[i].x : sca[i].y;
            const float sv = half_ok ? __builtin_amdgcn_cvt_f32_fp8((int)sw, blk & 3) : 0.0f;
            const f16x8 fa = dequant(ca[i][u], sv);
#pragma unroll
            for (int j = 0; j < SN; ++j)
              acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa, acc[j][i], 0, 0, 0);
          }
        });
      });
    } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (4 * t + s < ksteps) {
        // B fragments of the k-step stay in registers; each A fragment is
        // read just before its row of MFMAs
        v8i fb[SN];
#pragma unroll
        for (int j = 0; j < SN; ++j) fb[j] = frag(B, 32 * j + l32, s);
        // group-K: this lane's block past the group's k range scales to 0
        const bool blk_ok = !GK || (int64_t)(8 * t + 2 * s + h) * 32 < klen;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
          const v8i fa = frag(A, 32 * i + l32, s);
          const int sai = blk_ok ? pick(sca[i], s) : 0;
#pragma unroll
          for (int j = 0; j < SN; ++j)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa, acc[j][i], kE2M1, kE2M1, 0,
                                                                        blk_ok ? pick(scb[j], s) : 0, 0, sai);
        }
      }
    }
    }
    // this wave's DMA and scales landed (MXFP4: all but this k-tile's two
    // prefetch loads, so the previous k-tile's are in)
    if constexpr (NV) {
      if (more) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt2);
      // (an asm statement, so that the fold cannot move above the wait)
      asm volatile("v_add3_u32 %0, %0, %1, %2" : "+v"(pf_sink) : "v"(pf_prev[0]), "v"(pf_prev[1]));
    }
    if (more) {
      take_scales(t + 1, nsa, nsb);
    }
    __syncthreads();
  };
  // k-tile t_lo + j lives in stage j & 1
  for (int t = t_lo; t < t_hi; t += 2) {
    ktile(t, sA0, sB0, sA1, sB1, pf_even, pf_odd);
    if (t + 1 < t_hi) ktile(t + 1, sA1, sB1, sA0, sB0, pf_odd, pf_even);
  }
  asm volatile("" :: "v"(pf_sink ^ pf_even[0] ^ pf_even[1] ^ pf_odd[0] ^ pf_odd[1]));

  // lane l holds row 32 i + l32 and, per MFMA tile, columns 8 g + 4 h .. +3
  // (g = 0..3) in accumulator elements 4 g .. 4 g + 3. NVFP4: every product
  // still carries 1 / S of each operand's tensor (alpha, one rounding).
  const int64_t m0 = am0 + TM / 2 * wm, n0 = bn0 + TN / 2 * wn;
  float alpha = 1.0f;
  if constexpr (NV)
    alpha = (float)(1.0 / ((double)nvfp4_tensor_scale(*a_amax) * (double)nvfp4_tensor_scale(b_amax[grp])));
  if constexpr (SPLIT) {
    // a split-K part: the whole fp32 partial tile, row-major (pitch TN), into
    // its slot, through the wave's 32 KB LDS slice as whole 128-byte rows
    // (the staging of the fp32 epilogue below, without old values)
    uint8_t* const slice = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
    const float* wp = sp.ws + (int64_t)split_unit * TM * TN + (int64_t)(TM / 2 * wm) * TN + TN / 2 * wn;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(wp, ((int64_t)(TM / 2 - 1) * TN + TN / 2) * 4);
    const int rr = lane >> 3, cc = lane & 7;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      uint8_t* const st = slice + (i & 1) * (SN * 4096);
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x4 v;
          v.x = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 0]));
          v.y = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 1]));
          v.z = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 2]));
          v.w = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 3]));
          const int ch = 2 * g + h;
          *reinterpret_cast<u32x4*>(st + j * 4096 + l32 * 128 + ((ch ^ (l32 & 7)) << 4)) = v;
        }
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(st + j * 4096 + (8 * q + rr) * 128 + ((cc ^ rr) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(v, rd, ((uint32_t)(32 * i + 8 * q + rr) * TN + 32 * j + 4 * cc) * 4,
                                                 0, 2);
        }
    }
    return;
  } else {
  if (F32 && (N & 31) == 0 && N <= (1 << 22)) {
    // fp32 C leaves through the wave's 32 KB LDS slice (the operand stages
    // are free after the k-loop's last barrier) so that every store covers
    // whole 128-byte rows: 32 x 32 block (i, j) is staged as [row][16-byte
    // chunk], chunk c of row r at slot c ^ (r & 7), and read back so that lane
    // L holds row 8 q + L / 8, chunk L % 8 (q = 0..3). Old values of an
    // accumulating store are loaded in that layout, two 32-row blocks ahead.
    const int64_t wrows = min<int64_t>(TM / 2, row_end - m0);
    if (wrows <= 0) return;
    uint8_t* const slice = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
    const char* cb = reinterpret_cast<const char*>(c) + ((GK ? (int64_t)grp * M * N : 0) + m0 * N + n0) * 4;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(cb, wrows * N * 4);
    const uint32_t ld = (uint32_t)N;
    const int rr = lane >> 3, cc = lane & 7;
    const int jv = (int)min<int64_t>(SN, (N - n0) / 32);     // 32-column blocks inside C
    auto coff = [&](int i, int j, int q) __attribute__((always_inline)) -> uint32_t {
      return ((uint32_t)(32 * i + 8 * q + rr) * ld + 32 * j + 4 * cc) * 4;
    };
    constexpr int kOnce = 2;   // cache policy of memory touched once: non-temporal
    u32x4 old[2][SN][4];
    const bool acc_old = GK && accumulate;
    auto load_old = [&](int i, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) old[buf][j][q] = __builtin_amdgcn_raw_buffer_load_b128(rd, coff(i, j, q), 0, kOnce);
    };
    if (acc_old) {
      load_old(0, 0);
      load_old(1, 1);
    }
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      uint8_t* const st = slice + (i & 1) * (SN * 4096);
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x4 v;
          v.x = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 0]) * alpha);
          v.y = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 1]) * alpha);
          v.z = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 2]) * alpha);
          v.w = __float_as_uint(vgpr_hop(acc[j][i][4 * g + 3]) * alpha);
          const int ch = 2 * g + h;
          *reinterpret_cast<u32x4*>(st + j * 4096 + l32 * 128 + ((ch ^ (l32 & 7)) << 4)) = v;
        }
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        if (j < jv) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x4 v = *reinterpret_cast<const u32x4*>(st + j * 4096 + (8 * q + rr) * 128 + ((cc ^ rr) << 4));
            if (acc_old) {
              const u32x4 o = old[i & 1][j][q];
              v.x = __float_as_uint(__uint_as_float(v.x) + __uint_as_float(o.x));
              v.y = __float_as_uint(__uint_as_float(v.y) + __uint_as_float(o.y));
              v.z = __float_as_uint(__uint_as_float(v.z) + __uint_as_float(o.z));
              v.w = __float_as_uint(__uint_as_float(v.w) + __uint_as_float(o.w));
            }
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, coff(i, j, q), 0, kOnce);
          }
        }
      }
      if (acc_old && i + 2 < SM) load_old(i + 2, i & 1);
    }
    return;
  }
  }
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int64_t row = m0 + 32 * i + l32;
    if (row >= row_end) continue;
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = n0 + 32 * j + 8 * g + 4 * h;
        // through a VALU move, so the accumulators stay AGPR-only operands
        const float x0 = vgpr_hop(acc[j][i][4 * g]) * alpha, x1 = vgpr_hop(acc[j][i][4 * g + 1]) * alpha;
        const float x2 = vgpr_hop(acc[j][i][4 * g + 2]) * alpha, x3 = vgpr_hop(acc[j][i][4 * g + 3]) * alpha;
        if constexpr (F32) {
          float* cp = reinterpret_cast<float*>(c) + (GK ? (int64_t)grp * M * N : 0) + row * N + col;
          if (vec && col + 3 < N) {
            float4 v = make_float4(x0, x1, x2, x3);
            if (GK && accumulate) {
              const float4 o = *reinterpret_cast<const float4*>(cp);
              v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
            }
            *reinterpret_cast<float4*>(cp) = v;
          } else {
            const bool add = GK && accumulate;
            if (col < N) cp[0] = add ? cp[0] + x0 : x0;
            if (col + 1 < N) cp[1] = add ? cp[1] + x1 : x1;
            if (col + 2 < N) cp[2] = add ? cp[2] + x2 : x2;
            if (col + 3 < N) cp[3] = add ? cp[3] + x3 : x3;
          }
        } else {
          uint16_t* cp = reinterpret_cast<uint16_t*>(c) + row * N + col;
          if (vec && col + 3 < N) {
            *reinterpret_cast<uint2*>(cp) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
          } else {
            if (col < N) cp[0] = (uint16_t)bf16_rne(x0);
            if (col + 1 < N) cp[1] = (uint16_t)bf16_rne(x1);
            if (col + 2 < N) cp[2] = (uint16_t)bf16_rne(x2);
            if (col + 3 < N) cp[3] = (uint16_t)bf16_rne(x3);
          }
        }
      }
  }
}

// Split-K reduce: one workgroup per 16-row slab of a tail tile; a thread
// issues its loads (4 float4 positions x up to kMaxSplitParts parts) before
// adding the parts in part order, and writes C for the rows of the tile's
// group and the columns below N.
constexpr int kF4RedRows = 16;
template <bool F32>
__global__ __launch_bounds__(256) void fp4_split_reduce_kernel(Fp4Split sp, Fp4Groups gr, int64_t N,
                                                               int64_t n_tiles_n, void* c) {
  constexpr int TM = kFp4GemmTileM, TN = kFp4GemmTileN, kSlabs = TM / kF4RedRows;
  static_assert(kF4RedRows * TN == 4 * 4 * 256, "a slab is 4 float4 per thread");
  const int tile = (int)blockIdx.x / kSlabs, slab = (int)blockIdx.x % kSlabs;
  const int id = sp.first + tile;
  const int64_t mt = id / n_tiles_n, nt = id - mt * n_tiles_n;
  int lo = 0, hi = gr.n - 1;                  // the group of m-tile mt
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gr.tile0[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  const int64_t am0 = gr.row0[lo] + (mt - gr.tile0[lo]) * TM, row_end = gr.row0[lo + 1];
  const int64_t bn0 = nt * TN;
  const float* ws = sp.ws + (int64_t)tile * sp.parts * TM * TN + slab * kF4RedRows * TN;
  float4 v[kMaxSplitParts][4];
#pragma unroll
  for (int p = 0; p < kMaxSplitParts; ++p)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (p < sp.parts)
        v[p][k] = *reinterpret_cast<const float4*>(ws + (int64_t)p * TM * TN + (k * 256 + (int)threadIdx.x) * 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = (k * 256 + (int)threadIdx.x) * 4;
    const int64_t row = am0 + slab * kF4RedRows + e / TN, col = bn0 + e % TN;
    float4 sum = v[0][k];
#pragma unroll
    for (int p = 1; p < kMaxSplitParts; ++p)
      if (p < sp.parts) { sum.x += v[p][k].x; sum.y += v[p][k].y; sum.z += v[p][k].z; sum.w += v[p][k].w; }
    if (row >= row_end || col >= N) continue;
    const float x[4] = {sum.x, sum.y, sum.z, sum.w};
    if constexpr (F32) {
      float* cp = reinterpret_cast<float*>(c) + row * N + col;
      for (int q = 0; q < 4; ++q)
        if (col + q < N) cp[q] = x[q];
    } else {
      uint16_t* cp = reinterpret_cast<uint16_t*>(c) + row * N + col;
      for (int q = 0; q < 4; ++q)
        if (col + q < N) cp[q] = (uint16_t)bf16_rne(x[q]);
    }
  }
}

hipError_t launch_gemm_fp4(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           const Fp4Groups& gr, int64_t N, int64_t K, void* c, int32_t c_f32, hipStream_t stream,
                           const Fp4Split& split_in) {
  const int64_t tm = gr.tile0[gr.n], tn = (N + kFp4GemmTileN - 1) / kFp4GemmTileN;
  if (tm * tn == 0) return hipSuccess;
  Fp4KGroups kg{};
  const int64_t tiles = tm * tn;
  const bool split = split_in.parts > 1 && split_in.parts <= kMaxSplitParts && split_in.first >= 0 &&
                     split_in.first < tiles && split_in.ws != nullptr;
  const Fp4Split none{0, 0, nullptr};
  // whole tiles [0, first); with a split, the tail's parts in a launch of their own, then their sums
  const int64_t main_tiles = split ? split_in.first : tiles;
  if (main_tiles > 0) {
    if (c_f32)
      hipLaunchKernelGGL((gemm_fp4_kernel<false, true, false>), dim3((unsigned)main_tiles), dim3(256), 0, stream, a,
                         as, b, bs, gr, kg, (int64_t)0, N, K, tn, c, 0, nullptr, nullptr, none);
    else
      hipLaunchKernelGGL((gemm_fp4_kernel<false, false, false>), dim3((unsigned)main_tiles), dim3(256), 0, stream, a,
                         as, b, bs, gr, kg, (int64_t)0, N, K, tn, c, 0, nullptr, nullptr, none);
  }
  if (split) {
    const int64_t tail = tiles - split_in.first;
    hipLaunchKernelGGL((gemm_fp4_kernel<false, true, false, true>), dim3((unsigned)(tail * split_in.parts)),
                       dim3(256), 0, stream, a, as, b, bs, gr, kg, (int64_t)0, N, K, tn, nullptr, 0, nullptr,
                       nullptr, split_in);
    const dim3 rgrid((unsigned)(tail * (kFp4GemmTileM / kF4RedRows)));
    if (c_f32)
      hipLaunchKernelGGL(fp4_split_reduce_kernel<true>, rgrid, dim3(256), 0, stream, split_in, gr, N, tn, c);
    else
      hipLaunchKernelGGL(fp4_split_reduce_kernel<false>, rgrid, dim3(256), 0, stream, split_in, gr, N, tn, c);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(const uint8_t* a, const uint8_t* as, const float* a_amax, const uint8_t* b,
                             const uint8_t* bs, const float* b_amax, const Fp4Groups& gr, int64_t N, int64_t K,
                             void* c, int32_t c_f32, hipStream_t stream) {
  const int64_t tm = gr.tile0[gr.n], tn = (N + kFp4GemmTileN - 1) / kFp4GemmTileN;
  if (tm * tn == 0) return hipSuccess;
  Fp4KGroups kg{};
  if (c_f32)
    hipLaunchKernelGGL((gemm_fp4_kernel<false, true, true>), dim3((unsigned)(tm * tn)), dim3(256), 0, stream, a, as,
                       b, bs, gr, kg, (int64_t)0, N, K, tn, c, 0, a_amax, b_amax, Fp4Split{0, 0, nullptr});
  else
    hipLaunchKernelGGL((gemm_fp4_kernel<false, false, true>), dim3((unsigned)(tm * tn)), dim3(256), 0, stream, a, as,
                       b, bs, gr, kg, (int64_t)0, N, K, tn, c, 0, a_amax, b_amax, Fp4Split{0, 0, nullptr});
  return hipGetLastError();
}

hipError_t launch_gemm_fp4_group_k(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                                   const Fp4KGroups& kg, int64_t M, int64_t N, float* c, int32_t accumulate,
                                   hipStream_t stream) {
  const int64_t tm = (M + kFp4GemmTileM - 1) / kFp4GemmTileM, tn = (N + kFp4GemmTileN - 1) / kFp4GemmTileN;
  const int64_t tiles = (int64_t)kg.n * tm * tn;
  if (tiles == 0) return hipSuccess;
  Fp4Groups gr{};
  hipLaunchKernelGGL((gemm_fp4_kernel<true, true, false>), dim3((unsigned)tiles), dim3(256), 0, stream, a, as, b, bs,
                     gr, kg, M, N, kg.k0[kg.n], tn, c, accumulate, nullptr, nullptr, Fp4Split{0, 0, nullptr});
  return hipGetLastError();
}

}  // namespace mx
