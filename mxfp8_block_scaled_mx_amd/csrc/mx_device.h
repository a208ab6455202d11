// Device helpers shared by the MXFP8 kernels (gfx950).
//
// The block quantizer here is the one routine used by the standalone quantize
// kernel and by the GEMM epilogues that requantize fp32 intermediates, so both
// produce identical codes for identical inputs.
//
// MXFP8 block rule (one E8M0 scale per 32 consecutive values, E4M3 elements:
// "Efficient MoE training for biological foundation models", Key technical
// approaches item 2), with the scale exponent e = floor(log2 amax) - 8 clamped
// to [-127, 127] and saturating round-to-nearest-even elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// E8M0 scale code of a block from the bit pattern of its |amax| (finite fp32).
// floor(log2 amax) = biased exponent - 127 for normal amax, so
// code = e + 127 = biased - 8, clamped at 0; subnormal or zero amax -> 0.
__device__ __forceinline__ uint32_t scale_code_from_amax_bits(uint32_t amax_bits) {
  uint32_t eb = amax_bits >> 23;
  return eb > 8u ? eb - 8u : 0u;
}

// 2^(-e) = 2^(127 - code) as an fp32 (always a normal number for code <= 246).
__device__ __forceinline__ float inv_scale_from_code(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

__device__ __forceinline__ float clamp448(float t) {
  return fminf(fmaxf(t, -448.0f), 448.0f);
}

// Four fp32 values (already divided by the block scale) -> four E4M3 codes in
// one dword (byte i = value i). The hardware convert rounds to nearest even
// and keeps the sign of zero; clamping to +-448 first makes it saturating.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), lo, true);
  return (uint32_t)r;
}

__device__ __forceinline__ uint32_t abs_bits(float v) {
  return __float_as_uint(v) & 0x7FFFFFFFu;
}

// bf16 <-> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Cross-lane helpers (64-wide wavefront).
__device__ __forceinline__ uint32_t xor_u32(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, 64);
}
__device__ __forceinline__ float xor_f32(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// ---- cross-lane moves without LDS (DPP and the gfx950 permlane swaps)
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Half-wave exchange: lanes 0..31 send `lower_sends` to lane l + 32, lanes
// 32..63 send `upper_sends` to lane l - 32; returns what the lane received.
// (v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.)
__device__ __forceinline__ uint32_t xhalf(uint32_t lower_sends, uint32_t upper_sends, int h) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(upper_sends, lower_sends, false, false);
  return h ? r.x : r.y;
}
// max / sum of the values of lanes l and l ^ 32 (same on both lanes)
__device__ __forceinline__ uint32_t max_halves(uint32_t v) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(r.x, r.y);
}
__device__ __forceinline__ float sum_halves(float v) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

// Identity move through a VALU DPP instruction (quad_perm 0,1,2,3). Passing
// accumulator values through it before a plain store keeps the register
// allocator from treating the accumulators as either-class (AGPR or VGPR)
// operands of the store, which otherwise makes it evict them inside the
// main loop.
__device__ __forceinline__ float vgpr_hop(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xE4, 0xF, 0xF, false));
}

// ---- buffer resources and LDS DMA
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and never fault, which replaces per-lane row clamping at tile edges.
// Every field is made wave-uniform explicitly so the descriptor lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0xFFFFFFFFll;
  const uint32_t n = __builtin_amdgcn_readfirstlane((uint32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void* p = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, 0x00020000);
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) (resp. vmcnt(1)) with
// expcnt/lgkmcnt left open; issued through the builtin so the compiler's own
// waitcnt tracking knows the loads (and buffer->LDS DMA) have landed.
[[maybe_unused]] constexpr int kWaitVmcnt0 = 0x0F70;
[[maybe_unused]] constexpr int kWaitVmcnt1 = 0x0F71;

// Workgroups go to the 8 XCDs round-robin (block b runs on XCD b % 8). Tile
// ids are handed out in rounds of 8 x CHUNK: in each round XCD x takes
// CHUNK consecutive ids, so the tiles running together on one XCD are
// raster neighbours (they share A and B rows in that XCD's L2) while all XCDs
// walk the id space at the same pace, which keeps tiles of unequal cost
// (group-K slots sorted by size) balanced across XCDs. Blocks of the last,
// partial round keep their own id.
constexpr int kXcdChunk = 32;
template <int CHUNK = kXcdChunk>
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int round = 8 * CHUNK;
  const int full = total / round * round;
  if (bid >= full) return bid;
  const int xcd = bid & 7, local = bid >> 3;
  return (local / CHUNK) * round + xcd * CHUNK + local % CHUNK;
}

// Compile-time loop: fn(std::integral_constant<int, i>) for i in [I, N). Keeps
// register-array indices constant however large the body is.
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

}  // namespace mx
