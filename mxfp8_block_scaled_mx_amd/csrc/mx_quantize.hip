// MXFP8 quantize kernel for gfx950: one pass over a bf16/fp32 matrix writes
// the rowwise copy straight from registers and the columnwise copy through an
// LDS transpose (one E8M0 scale per 32 consecutive values along the row, resp.
// along the column: "Efficient MoE training for biological foundation models",
// Key technical approaches item 2).
//
// Tile: 128 rows x 256 bytes of input (128 bf16 or 64 fp32 columns), 256
// threads. Each thread loads 16 contiguous bytes per pass (a 16-thread row
// segment is 256 contiguous bytes, fully coalesced); the 4 (bf16) or 8 (fp32)
// threads of one 32-block reduce their amax with two or three xor shuffles.
// The tile is staged in LDS unchanged; the columnwise phase then reads 32
// values down each column (consecutive lanes read consecutive dwords of one
// LDS row, conflict-free) and writes 32 contiguous code bytes per column.
// Row tiles restart at each group's first row so columnwise blocks never
// straddle groups; rows past the group's end are zeros (padding codes 0x00).
// Scales go to the row-major layout or, for the fused MLP's internal
// buffers, to the k-tiled layout (see ScaleStrides).
#include "mx_device.h"
#include "mx_internal.h"

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

// Offset of the rowwise scale of (row r, block b) in the row-major or
// k-tiled layout.
__device__ __forceinline__ int64_t row_scale_offset(const QuantArgs& args, int64_t r, int b) {
  if (args.tiled) return ((r >> 5) * args.nq_row + (b >> 2)) * 128 + (r & 31) * 4 + (b & 3);
  return r * (args.cols / 32) + b;
}

template <typename T>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs args) {
  constexpr int VPT = QTraits<T>::kVals;
  constexpr int TC = QTraits<T>::kCols;
  constexpr int TR = kQuantTileRows;
  constexpr int TPB = 32 / VPT;  // threads per 32-block along a row
  __shared__ __attribute__((aligned(16))) uint8_t tile[TR * 256];

  const int tid = threadIdx.x;
  const int ct = blockIdx.x % args.n_col_tiles;
  const int rt_global = blockIdx.x / args.n_col_tiles;

  // group of this row tile
  int g = 0;
  {
    int lo = 0, hi = args.groups.n - 1;
    while (lo < hi) {  // last g with tile0[g] <= rt_global
      int mid = (lo + hi + 1) >> 1;
      if (args.groups.tile0[mid] <= rt_global) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
  const int rt = rt_global - args.groups.tile0[g];
  const int64_t grow0 = args.groups.row0[g];
  const int m_g = args.groups.row0[g + 1] - args.groups.row0[g];
  const int tile_r0 = rt * TR;                 // first row of the tile within the group
  const int64_t cols = args.cols;
  const int col_base = ct * TC;

  const T* x = reinterpret_cast<const T*>(args.x);
  const int cc = tid & 15;                     // 16-byte chunk within the row segment
  const int col = col_base + cc * VPT;
  const bool col_ok = col < cols;

#pragma unroll 2
  for (int p = 0; p < TR / 16; ++p) {
    const int r = p * 16 + (tid >> 4);
    const bool row_ok = (tile_r0 + r) < m_g;
    uint4 raw = make_uint4(0, 0, 0, 0);
    const int64_t grow = grow0 + tile_r0 + r;
    if (row_ok && col_ok) raw = *reinterpret_cast<const uint4*>(x + grow * cols + col);
    *reinterpret_cast<uint4*>(tile + r * 256 + cc * 16) = raw;
    if (args.q_row != nullptr) {
      float v[VPT];
      unpack16<T>(raw, v);
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
        if ((cc % TPB) == 0) args.s_row[row_scale_offset(args, grow, col / 32)] = (uint8_t)sc;
      } else if (args.tiled && col_ok && (cc % TPB) == 0 && grow >= args.rows && grow < ((args.rows + 31) & ~31)) {
        // k-tiled: the pad rows of the last 32-row group get scale 0 (2^-127)
        args.s_row[row_scale_offset(args, grow, col / 32)] = 0;
      }
    }
  }
  if (args.q_col == nullptr) return;
  __syncthreads();

  // columnwise: unit = (column slot, 32-row block); 4 row blocks x 64 slots
  const int rb = tid >> 6;
  const int slot = tid & 63;
  if (tile_r0 + rb * 32 >= m_g) return;        // block entirely past the group: not in the layout
  const int64_t qc0 = args.groups.pcol0[g] + tile_r0 + rb * 32;
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
#pragma unroll
  for (int c = 0; c < CPS; ++c) {
    const int64_t colc = col_base + slot * CPS + c;
    if (colc >= cols) continue;
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
    uint8_t* qd = args.q_col + colc * args.ld_col + qc0;
    *reinterpret_cast<uint4*>(qd) = w0;
    *reinterpret_cast<uint4*>(qd + 16) = w1;
    if (args.tiled) {
      const int bl = (tile_r0 + rb * 32) >> 5;       // block index inside the group
      args.s_col[((colc >> 5) * args.nq_col + args.groups.q0[g] + (bl >> 2)) * 128 + (colc & 31) * 4 + (bl & 3)] =
          (uint8_t)sc;
    } else {
      args.s_col[colc * (args.ld_col / 32) + qc0 / 32] = (uint8_t)sc;
    }
  }
}

hipError_t launch_quantize(const QuantArgs& args, int x_dtype, int total_row_tiles, hipStream_t stream) {
  const int64_t blocks = (int64_t)total_row_tiles * args.n_col_tiles;
  if (blocks == 0) return hipSuccess;
  if (x_dtype == MX_BF16)
    hipLaunchKernelGGL(quantize_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream, args);
  else
    hipLaunchKernelGGL(quantize_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mx
