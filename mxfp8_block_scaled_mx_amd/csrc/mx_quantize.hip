// MXFP8 quantize kernel for gfx950: one pass over a bf16/fp32 matrix writes
// the rowwise copy straight from registers and the columnwise copy through an
// LDS transpose (one E8M0 scale per 32 consecutive values along the row, resp.
// along the column: "Efficient MoE training for biological foundation models",
// Key technical approaches item 2).
//
// Tile: 128 rows x 256 bytes of input (128 bf16 or 64 fp32 columns), 256
// threads. Each thread issues all 8 of its 16-byte loads first (a 16-thread
// row segment is 256 contiguous bytes); the 4 (bf16) or 8 (fp32) threads of
// one 32-block reduce their amax with two or three xor shuffles and store the
// rowwise codes directly. The tile is staged in LDS unchanged; the columnwise
// phase reads 32 values down each column (consecutive lanes read consecutive
// dwords of one LDS row, conflict-free), stages the codes as [column][row] in
// LDS and writes each column's 128 tile rows as one run. Scales of a row (a
// column) within the tile are gathered into one word, so the k-tiled layout
// receives whole 128-byte lines.
// Row tiles restart at each group's first row so columnwise blocks never
// straddle groups; rows past the group's end are zeros (padding codes 0x00).
// Scales go to the row-major layout or, for the fused MLP's internal
// buffers, to the k-tiled layout (see ScaleStrides).
#include "mx_device.h"
#include "mx_internal.h"

#include <algorithm>

namespace mx {

template <typename T>
struct QTraits;
template <>
struct QTraits<uint16_t> {  // bf16
  static constexpr int kVals = 8;           // values per 16-byte chunk
  static constexpr int kCols = 128;         // tile columns
};
template <>
struct QTraits<float> {
  static constexpr int kVals = 4;
  static constexpr int kCols = 64;
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& raw, float* v);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& raw, float* v) {
  v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
  v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
  v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
  v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
}
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& raw, float* v) {
  v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
  v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
}

template <bool DEVG>
__device__ __forceinline__ const QuantGroups& quant_groups(const QuantArgs& a) {
  if constexpr (DEVG) return *a.groups_dev;
  else return a.groups;
}

template <typename T, bool DEVG>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs args) {
  constexpr int VPT = QTraits<T>::kVals;
  constexpr int TC = QTraits<T>::kCols;
  constexpr int TR = kQuantTileRows;
  constexpr int TPB = 32 / VPT;              // threads per 32-block along a row
  constexpr int NB = TC / 32;                // 32-blocks per tile row (4 bf16, 2 f32)
  __shared__ __attribute__((aligned(16))) uint8_t tile[TR * 256];   // input tile, as loaded
  // columnwise codes [column][row], in the input tile's memory once the
  // columns are in registers; the 16-byte pad per column spreads the 16-byte
  // writes of consecutive column pairs over the LDS banks
  constexpr int CST = TR + 16;
  static_assert(TC * CST <= TR * 256, "columnwise staging must fit the input tile");
  uint8_t* const ctile = tile;
  __shared__ uint8_t rs_t[TR * 4];           // rowwise scales [row][block]
  __shared__ uint8_t cs_t[TC * 4];           // columnwise scales [column][block]

  const QuantGroups& G = quant_groups<DEVG>(args);
  // a device-built table covers fewer row tiles than the worst-case grid
  if constexpr (DEVG)
    if ((int)blockIdx.x / args.n_col_tiles >= G.tile0[G.n]) return;
  const int tid = threadIdx.x;
  const int cc = tid & 15;                     // 16-byte chunk within the row segment
  const int64_t cols = args.cols;
  const T* x = reinterpret_cast<const T*>(args.x);

  struct Loc {
    int g, tile_r0, m_g, col_base;
    int64_t grow0;
  };
  auto locate = [&](int t) __attribute__((always_inline)) -> Loc {
    Loc L;
    const int ct = t % args.n_col_tiles;
    const int rt_global = t / args.n_col_tiles;
    int lo = 0, hi = G.n - 1;        // last group with tile0 <= rt_global
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (G.tile0[mid] <= rt_global) lo = mid; else hi = mid - 1;
    }
    L.g = lo;
    L.tile_r0 = (rt_global - G.tile0[lo]) * TR;   // first row of the tile within the group
    L.grow0 = G.row0[lo];
    L.m_g = G.row0[lo + 1] - G.row0[lo];
    L.col_base = ct * TC;
    return L;
  };
  // the tile's 8 x 16 bytes per thread, all requested at once
  auto load = [&](const Loc& L, uint4 (&raw)[TR / 16]) __attribute__((always_inline)) {
    const int col = L.col_base + cc * VPT;
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int r = p * 16 + (tid >> 4);
      raw[p] = make_uint4(0, 0, 0, 0);
      if ((L.tile_r0 + r) < L.m_g && col < cols) {
        int64_t src = L.grow0 + L.tile_r0 + r;
        if (args.row_index != nullptr) {
          src = args.row_index[src];
          if (src < 0 || src >= args.index_rows) continue;
        }
        raw[p] = *reinterpret_cast<const uint4*>(x + src * cols + col);
      }
    }
  };
  auto process = [&](const Loc& L, const uint4 (&raw)[TR / 16]) __attribute__((always_inline)) {
    const int g = L.g, tile_r0 = L.tile_r0, m_g = L.m_g, col_base = L.col_base;
    const int64_t grow0 = L.grow0;
    const int col = col_base + cc * VPT;
    const bool col_ok = col < cols;
#pragma unroll
    for (int p = 0; p < TR / 16; ++p) {
      const int r = p * 16 + (tid >> 4);
      const bool row_ok = (tile_r0 + r) < m_g;
      const int64_t grow = grow0 + tile_r0 + r;
      *reinterpret_cast<uint4*>(tile + r * 256 + cc * 16) = raw[p];
      if (args.q_row != nullptr) {
        float v[VPT];
        unpack16<T>(raw[p], v);
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < VPT; ++i) am = umax(am, abs_bits(v[i]));
#pragma unroll
        for (int s = 1; s < TPB; s <<= 1) am = umax(am, xor_u32(am, s));
        const uint32_t sc = scale_code_from_amax_bits(am);
        const float inv = inv_scale_from_code(sc);
        if (row_ok && col_ok) {
          uint8_t* qd = args.q_row + grow * cols + col;
          if constexpr (VPT == 8) {
            uint2 w;
            w.x = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            w.y = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
            *reinterpret_cast<uint2*>(qd) = w;
          } else {
            *reinterpret_cast<uint32_t*>(qd) = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
          }
        }
        if ((cc % TPB) == 0) rs_t[r * 4 + cc / TPB] = (uint8_t)sc;
      }
    }
    __syncthreads();

    // rowwise scales of the tile: one word (the tile's blocks) per row
    if (args.q_row != nullptr && tid < TR) {
      const int r = tid;
      const int64_t grow = grow0 + tile_r0 + r;
      const uint32_t word = *reinterpret_cast<const uint32_t*>(rs_t + r * 4);
      const int b0 = col_base / 32;             // first block of the tile in the row
      if (tile_r0 + r < m_g) {
        if (args.tiled) {
          uint8_t* sd = args.s_row + ((grow >> 5) * args.nq_row + (b0 >> 2)) * 128 + (grow & 31) * 4 + (b0 & 3);
          if constexpr (NB == 4) *reinterpret_cast<uint32_t*>(sd) = word;
          else *reinterpret_cast<uint16_t*>(sd) = (uint16_t)word;
        } else if (NB == 4 && (cols & 127) == 0 && (reinterpret_cast<uintptr_t>(args.s_row) & 3) == 0) {
          // row-major, whole 128-column tile: its 4 scale bytes as one aligned word
          *reinterpret_cast<uint32_t*>(args.s_row + grow * (cols / 32) + b0) = word;
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (col_base + 32 * j < cols) args.s_row[grow * (cols / 32) + b0 + j] = (uint8_t)(word >> (8 * j));
        }
      } else if (args.tiled && grow >= args.rows && grow < ((args.rows + 31) & ~31)) {
        // k-tiled: the pad rows of the last 32-row group get scale 0 (2^-127)
        uint8_t* sd = args.s_row + ((grow >> 5) * args.nq_row + (b0 >> 2)) * 128 + (grow & 31) * 4 + (b0 & 3);
        if constexpr (NB == 4) *reinterpret_cast<uint32_t*>(sd) = 0;
        else *reinterpret_cast<uint16_t*>(sd) = 0;
      }
    }
    if (args.q_col != nullptr) {
    // columnwise: unit = (column slot, 32-row block); 4 row blocks x 64 slots.
    // Codes go to ctile[column][row], scales to cs_t[column][block].
    {
      const int rb = tid >> 6;
      const int slot = tid & 63;
      constexpr int CPS = 4 / sizeof(T) > 0 ? 4 / (int)sizeof(T) : 1;  // columns per dword
      float v[CPS][32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(tile + (rb * 32 + i) * 256 + slot * 4);
        if constexpr (CPS == 2) {
          v[0][i] = bf16_lo(w);
          v[1][i] = bf16_hi(w);
        } else {
          v[0][i] = __uint_as_float(w);
        }
      }
      __syncthreads();                           // every column read: the tile becomes ctile
#pragma unroll
      for (int c = 0; c < CPS; ++c) {
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) am = umax(am, abs_bits(v[c][i]));
        const uint32_t sc = scale_code_from_amax_bits(am);
        const float inv = inv_scale_from_code(sc);
        uint4 w0, w1;
        w0.x = e4m3x4(v[c][0] * inv, v[c][1] * inv, v[c][2] * inv, v[c][3] * inv);
        w0.y = e4m3x4(v[c][4] * inv, v[c][5] * inv, v[c][6] * inv, v[c][7] * inv);
        w0.z = e4m3x4(v[c][8] * inv, v[c][9] * inv, v[c][10] * inv, v[c][11] * inv);
        w0.w = e4m3x4(v[c][12] * inv, v[c][13] * inv, v[c][14] * inv, v[c][15] * inv);
        w1.x = e4m3x4(v[c][16] * inv, v[c][17] * inv, v[c][18] * inv, v[c][19] * inv);
        w1.y = e4m3x4(v[c][20] * inv, v[c][21] * inv, v[c][22] * inv, v[c][23] * inv);
        w1.z = e4m3x4(v[c][24] * inv, v[c][25] * inv, v[c][26] * inv, v[c][27] * inv);
        w1.w = e4m3x4(v[c][28] * inv, v[c][29] * inv, v[c][30] * inv, v[c][31] * inv);
        const int cl = slot * CPS + c;           // column inside the tile
        *reinterpret_cast<uint4*>(ctile + cl * CST + rb * 32) = w0;
        *reinterpret_cast<uint4*>(ctile + cl * CST + rb * 32 + 16) = w1;
        cs_t[cl * 4 + rb] = (uint8_t)sc;
      }
    }
    __syncthreads();

    // Columnwise codes: each column's 128 tile rows are one contiguous run of the
    // layout; 8 lanes x 16 bytes per column. Blocks past the group's end are not
    // part of the layout (the next group's columns start there).
    const int64_t qc0 = G.pcol0[g] + tile_r0;
#pragma unroll
    for (int it = 0; it < TC * 8 / 256; ++it) {
      const int c = it * 256 + tid;
      const int cl = c >> 3, part = c & 7;
      const int64_t colc = col_base + cl;
      const uint4 w = *reinterpret_cast<const uint4*>(ctile + cl * CST + part * 16);
      if (colc < cols && tile_r0 + 32 * (part >> 1) < m_g)
        *reinterpret_cast<uint4*>(args.q_col + colc * args.ld_col + qc0 + part * 16) = w;
    }
    // columnwise scales: one word (the tile's 4 blocks) per column
    if (tid < TC) {
      const int cl = tid;
      const int64_t colc = col_base + cl;
      if (colc < cols) {
        uint32_t word = *reinterpret_cast<const uint32_t*>(cs_t + cl * 4);
        if (args.tiled) {
          // blocks past the group's end in its last step are cleared
          const int nvalid = (m_g - tile_r0 + 31) >> 5;
          if (nvalid < 4) word &= (1u << (8 * nvalid)) - 1u;
          *reinterpret_cast<uint32_t*>(args.s_col + ((colc >> 5) * args.nq_col + G.q0[g] + (tile_r0 >> 7)) * 128 +
                                       (colc & 31) * 4) = word;
        } else if (tile_r0 + 96 < m_g && ((args.ld_col | qc0) & 127) == 0 &&
                   (reinterpret_cast<uintptr_t>(args.s_col) & 3) == 0) {
          // row-major, all 4 blocks inside the group: one aligned word
          *reinterpret_cast<uint32_t*>(args.s_col + colc * (args.ld_col / 32) + qc0 / 32) = word;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (tile_r0 + 32 * j < m_g) args.s_col[colc * (args.ld_col / 32) + qc0 / 32 + j] = (uint8_t)(word >> (8 * j));
        }
      }
    }
    }
    };

  const Loc cur = locate(blockIdx.x);
  uint4 raw[TR / 16];
  load(cur, raw);
  process(cur, raw);
}

hipError_t launch_quantize(const QuantArgs& args, int x_dtype, int total_row_tiles, hipStream_t stream) {
  const int64_t blocks = (int64_t)total_row_tiles * args.n_col_tiles;
  if (blocks == 0) return hipSuccess;
  if (args.groups_dev != nullptr) {
    if (x_dtype != MX_BF16) return hipErrorInvalidValue;
    hipLaunchKernelGGL((quantize_kernel<uint16_t, true>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
  } else if (x_dtype == MX_BF16) {
    hipLaunchKernelGGL((quantize_kernel<uint16_t, false>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
  } else {
    hipLaunchKernelGGL((quantize_kernel<float, false>), dim3((unsigned)blocks), dim3(256), 0, stream, args);
  }
  return hipGetLastError();
}

// Plain device copy (the HBM reference of the casts): every thread moves 4 x 16
// bytes per pass, all loads issued before the stores; loads and stores are
// non-temporal (each byte is touched once).
__global__ __launch_bounds__(256) void device_copy_kernel(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n16; base += step) {
    v4i v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + 256 * i < n16) v[i] = __builtin_nontemporal_load(src + base + 256 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + 256 * i < n16) __builtin_nontemporal_store(v[i], dst + base + 256 * i);
  }
}

hipError_t launch_device_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + 1023) / 1024, 256 * 16);
  hipLaunchKernelGGL(device_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const v4i*>(src), reinterpret_cast<v4i*>(dst), n16);
  return hipGetLastError();
}

}  // namespace mx
