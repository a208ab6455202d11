// Rowwise MXFP4 cast: E2M1 elements with one E8M0 scale per 32 consecutive
// values (the MX block format the pages name next to MXFP8, run at 4 bits on
// MI355X: "examples/llama: default-on fusion & DP-comm perf toggles", the
// mxfp4 Llama runs). Scale exponent floor(log2 amax) - 2 (2 = exponent of
// E2M1's largest value, 6); element = nearest E2M1 value of v / 2^e, ties to
// the even code, saturating at 6; two codes per byte, element 2i in the low
// nibble.
//
// Rowwise: one thread per 32-value block: four 16-byte loads, a local amax,
// the scale code from the amax exponent bits, the elements scaled by 2^-e
// (exact) and rounded by comparing against the midpoints of the E2M1 grid, 16
// bytes of codes stored at once. Columnwise: see the columnwise kernel.
// HBM-bound.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// E2M1 code of |t| (exact, already scaled), ties to the even code: the
// midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 each either belong to the
// lower code (its code is even) or the upper one.
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fabsf(t);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return c | ((__float_as_uint(t) >> 28) & 8u);
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
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = umax(am, abs_bits(v[i]));
  // code = floor(log2 amax) - 2 + 127 = biased exponent - 2, clamped at 0
  // (zero or subnormal amax, or a biased exponent below 3)
  const uint32_t eb = am >> 23;
  const uint32_t sc = eb > 2u ? eb - 2u : 0u;
  const float inv = inv_scale_from_code(sc);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= e2m1_code(v[8 * i + j] * inv) << (4 * j);
    w[i] = word;
  }
  *reinterpret_cast<uint4*>(q + r * (cols / 2) + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  s[r * nb + b] = (uint8_t)sc;
}

// Columnwise MXFP4 (= rowwise of the transpose): codes [cols, rows/2] and
// scales [cols, rows/32]; rows % 32 == 0. A workgroup stages a 128-row x
// 64-column tile in LDS (rows loaded as coalesced 16-byte pieces); thread t
// then takes column t % 64 and the 32-row block t / 64, reduces the block's
// amax locally and stores its 16 code bytes as one piece of the column's run.
constexpr int kFp4ColTileRows = 128, kFp4ColTileCols = 64;
__global__ __launch_bounds__(256) void quantize_fp4_colwise_kernel(const uint16_t* x, int64_t rows, int64_t cols,
                                                                   uint8_t* q, uint8_t* s) {
  // [row][column] bf16 with a 2-element pad so that the column reads of a
  // wave (64 columns of one row) spread over the banks
  __shared__ uint16_t tile[kFp4ColTileRows][kFp4ColTileCols + 2];
  const int64_t n_ct = (cols + kFp4ColTileCols - 1) / kFp4ColTileCols;
  const int64_t r0 = (int64_t)(blockIdx.x / n_ct) * kFp4ColTileRows;
  const int64_t c0 = (int64_t)(blockIdx.x % n_ct) * kFp4ColTileCols;
  const int tid = threadIdx.x;
  // 128 rows x 8 pieces of 16 bytes (8 columns each): 4 pieces per thread
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
  const int c = tid % kFp4ColTileCols, rb = tid / kFp4ColTileCols;
  const int64_t col = c0 + c, row = r0 + 32 * rb;
  if (col >= cols || row >= rows) return;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float((uint32_t)tile[32 * rb + i][c] << 16);
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = umax(am, abs_bits(v[i]));
  const uint32_t eb = am >> 23;
  const uint32_t sc = eb > 2u ? eb - 2u : 0u;
  const float inv = inv_scale_from_code(sc);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) word |= e2m1_code(v[8 * i + j] * inv) << (4 * j);
    w[i] = word;
  }
  *reinterpret_cast<uint4*>(q + col * (rows / 2) + row / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  s[col * (rows / 32) + row / 32] = (uint8_t)sc;
}

hipError_t launch_quantize_fp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                               uint8_t* s_col, hipStream_t stream) {
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
  const int64_t blocks = q != nullptr ? rows * (cols / 32) : 0;
  if (blocks > 0)
    hipLaunchKernelGGL(quantize_fp4_rowwise_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, stream,
                       xb, rows, cols, q, s);
  if (q_col != nullptr && rows > 0) {
    const int64_t tiles = ((rows + kFp4ColTileRows - 1) / kFp4ColTileRows) *
                          ((cols + kFp4ColTileCols - 1) / kFp4ColTileCols);
    hipLaunchKernelGGL(quantize_fp4_colwise_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, xb, rows, cols,
                       q_col, s_col);
  }
  return hipGetLastError();
}

}  // namespace mx
