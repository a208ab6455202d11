// Grouped block-scaled GEMM on gfx950's scaled FP8 MFMA
// (V_MFMA_SCALE_F32_32X32X64_F8F6F4), C[m, n] = sum_k A[m, k] B[n, k] with
// both operands K-contiguous MXFP8 (E4M3 codes + one E8M0 scale per 32 k).
//
// GroupedLinear over per-expert split_sizes is one launch over a flat tile
// list ("Efficient MoE training for biological foundation models", Key
// technical approaches item 1); the SwiGLU / routing-weight / requantize
// epilogues realise the fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear
// forward and its backward (item 3).
//
// Tiling: 256 (A rows, "m") x 256 (B rows, "n") x 128 (k) per workgroup of
// 256 threads = 4 waves in 2 (m) x 2 (n), one wave per SIMD so each wave can
// keep its 256 fp32 accumulators in AGPRs. A wave owns m rows [128*wm, +128)
// and the four 32-row n sub-tiles {64*wn, 64*wn+32, 128+64*wn, 160+64*wn},
// i.e. 4 x 4 MFMA tiles of 32x32. The MFMA's first operand is the B tile
// (n), its second the A tile (m), so each lane ends up with one m row
// (lane % 32) and 16 n values: 4 runs of 4 consecutive n. With the SwiGLU
// pairing (tile rows 0..127 = gate rows, 128..255 = the matching up rows)
// sub-tiles s and s+2 hold gate and up of the same (row, j) in the same
// accumulator slot, and the 32 j's of one MXFP8 block sit in lanes l, l^32.
//
// Operand layout inside the MFMA (pinned on hardware): lane l = row (l%32),
// half h = l/32 holds k [16h, 16h+16) in bytes 0-15 and k [32+16h, +16) in
// bytes 16-31 of its 32-byte operand; the scale register of lane l (byte 0)
// scales k-block h of its row.
//
// LDS: double-buffered A and B tiles, 128 bytes per row, 16-byte chunk c of
// row r stored at chunk (c ^ ((r >> 1) & 7)): the 16 rows one ds_read_b128
// phase reads (16 lanes x 16 bytes over the 64 banks) then land in 16
// distinct 16-byte bank groups. Global loads go through registers
// one k-step ahead of the MFMAs (scalar base + 32-bit per-lane offsets).
// Scales are read straight from global memory (L2-resident), also one step
// ahead.
//
// Tile order: workgroup ids are first spread evenly over the 8 XCDs (ids that
// run on one XCD form one contiguous range of tiles, which then share its L2),
// then mapped to (group, m-tile, n-tile) with m-tiles grouped in bands of 8
// so the tiles in flight reuse the same A rows and B rows.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

constexpr int BM = kTileM, BN = kTileN, BK = kTileK;
constexpr int kThreads = 256;
constexpr int kBandM = 8;
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt/lgkmcnt left
// open; issued through the builtin so the compiler's own waitcnt tracking
// knows the loads have landed.
constexpr int kWaitVmcnt0 = 0x0F70;

struct TileCoord {
  int slot;   // group slot in the table
  int mt, nt; // tile indices within the group
};

__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

__device__ __forceinline__ TileCoord locate_tile(const GemmGroups& gt, int id, int mode, int M, int n_tiles_n) {
  int lo = 0, hi = gt.n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (gt.tile0[mid] <= id) lo = mid; else hi = mid - 1;
  }
  TileCoord t;
  t.slot = lo;
  const int local = id - gt.tile0[lo];
  const int rows = mode == MX_GROUP_M ? gt.len[lo] : M;
  const int mtiles = (rows + BM - 1) / BM;
  // band raster: kBandM m-tiles x all n-tiles, m fastest inside a band
  const int per_band = kBandM * n_tiles_n;
  const int band = local / per_band;
  const int in_band = local - band * per_band;
  const int band_m0 = band * kBandM;
  const int band_h = min(kBandM, mtiles - band_m0);
  t.mt = band_m0 + in_band % band_h;
  t.nt = in_band / band_h;
  return t;
}

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

template <int MODE, int EPI, bool SVEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs args, int total_tiles) {
  // The body uses gfx950-only types and builtins (buffer resources, LDS DMA);
  // the host compilation pass only needs the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  // Two stages of A and B tiles as four separate LDS objects: with the stage
  // index a compile-time constant the compiler can see that the DMA into one
  // stage never aliases the ds_reads of the other, so it does not wait for
  // the in-flight loads before computing.
  __shared__ __attribute__((aligned(16))) uint8_t sA0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[BN * BK];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[BN * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int id = xcd_remap(blockIdx.x, total_tiles);
  const TileCoord tc = locate_tile(args.groups, id, MODE, args.M, args.n_tiles_n);
  const int slot = tc.slot;
  const int g = args.groups.gid[slot];

  // ---- geometry of this tile
  int64_t a_row0;     // first global A row of the tile
  int a_rows_valid;   // rows of A valid in this tile (from a_row0)
  int64_t kbeg;       // first k column
  int klen;           // k columns to contract (multiple of 32)
  int b_rows;         // rows of B_g
  const uint8_t* bq = args.b;
  const uint8_t* bsc = args.bs;
  if constexpr (MODE == MX_GROUP_M) {
    a_row0 = (int64_t)args.groups.a0[slot] + (int64_t)tc.mt * BM;
    a_rows_valid = args.groups.len[slot] - tc.mt * BM;
    kbeg = 0;
    klen = args.K;
    bq += (int64_t)g * args.b_group_stride;
    bsc += (int64_t)g * (args.b_group_stride / 32);
  } else {
    a_row0 = (int64_t)tc.mt * BM;
    a_rows_valid = args.M - tc.mt * BM;
    kbeg = args.groups.a0[slot];
    klen = args.groups.len[slot];
  }
  b_rows = EPI == EPI_SWIGLU_FWD ? 2 * args.F : args.N;
  if (a_rows_valid > BM) a_rows_valid = BM;
  const int nk = (klen + BK - 1) / BK;
  const uint32_t lda = (uint32_t)args.lda, ldb = (uint32_t)args.ldb;
  const uint32_t lds_a = lda / 32, lds_b = ldb / 32;
  const int blk_last = (int)((kbeg + klen) / 32) - 1;  // last valid k block (clamp target)

  // Operand tiles through buffer resources: rows past the valid ones read as 0.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.a + a_row0 * lda + kbeg, (int64_t)(a_rows_valid - 1) * lda + klen);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + kbeg, (int64_t)(b_rows - 1) * ldb + klen);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(args.as + a_row0 * lds_a, (int64_t)a_rows_valid * lds_a);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bsc, (int64_t)b_rows * lds_b);

  // first B row of tile row block r0 (a multiple of 8 rows): SwiGLU fwd pairs
  // gate rows [nt*128, +128) (tile rows 0..127) with up rows F + the same j
  auto b_row_base = [&](int r0) __attribute__((always_inline)) -> uint32_t {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      return (uint32_t)((r0 < BN / 2) ? tc.nt * (BN / 2) + r0 : args.F + tc.nt * (BN / 2) + (r0 - BN / 2));
    else
      return (uint32_t)(tc.nt * BN + r0);
  };
  auto nsub = [&](int s) __attribute__((always_inline)) -> int { return (s < 2 ? 64 * wn + 32 * s : BN / 2 + 64 * wn + 32 * (s - 2)); };

  // ---- direct buffer->LDS loads: per k-step each wave fills 8 blocks of 1 KB
  // (8 tile rows) of A and of B; LDS slot = lane, i.e. row r = 8*blk + lane/8
  // and stored chunk lane%8, which holds logical chunk
  // (lane%8) ^ ((r >> 1) & 7) = (lane%8) ^ (lane/16) ^ 4*(blk&1), and
  // blk&1 = wave&1 for every blk this wave loads.
  const int lch = (lane & 7) ^ (lane >> 4) ^ (4 * (wave & 1));   // logical chunk this lane fetches
  const uint32_t va_off = (uint32_t)(lane >> 3) * lda + lch * 16;
  const uint32_t vb_off = (uint32_t)(lane >> 3) * ldb + lch * 16;
  const uint32_t vsa_off = (uint32_t)l32 * lds_a;
  const uint32_t vsb_off = (uint32_t)l32 * lds_b;

  v16f acc[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][mi][v] = 0.0f;

  // scales: raw words (dword path) or bytes of the next and current k-step
  uint32_t sb_n[4][2], sa_n[4][2];
  uint32_t sb_c[4][2], sa_c[4][2];

  // Scale loads of one k-step, in 8 slices (slice p: sub-tile p of B for
  // p < 4, m sub-tile p-4 of A after), so they spread over the 8 MFMA steps.
  auto load_scale_part = [&](int k0, int p) __attribute__((always_inline)) {
    const int blk0 = (int)((kbeg + k0) / 32);
    const __amdgpu_buffer_rsrc_t& rs = p < 4 ? rsb : rsa;
    const uint32_t voff = p < 4 ? vsb_off : vsa_off;
    const uint32_t so = p < 4 ? b_row_base(nsub(p)) * lds_b : (uint32_t)(128 * wm + 32 * (p - 4)) * lds_a;
    uint32_t* dst = p < 4 ? sb_n[p] : sa_n[p - 4];
    if constexpr (SVEC) {
      dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, so + blk0, 0);
      dst[1] = 0;
    } else {
      // per-lane block index: blk0 + h (+2), clamped to the group's last block
      const uint32_t b0 = (uint32_t)min(blk0 + h, blk_last), b1 = (uint32_t)min(blk0 + 2 + h, blk_last);
      dst[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff + b0, so, 0);
      dst[1] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff + b1, so, 0);
    }
  };
  // Slice p (0..7) of the loads of k-step kt: one 1 KB block (8 tile rows) of
  // A and of B into the LDS stage, and one scale slice into registers.
  auto load_part = [&](int kt, uint8_t* dA, uint8_t* dB, int p) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const int blk = p * 4 + wave;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dA + blk * 1024), 16, va_off,
                                             (uint32_t)(8 * blk) * lda + k0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dB + blk * 1024), 16, vb_off,
                                             b_row_base(8 * blk) * ldb + k0, 0, 0);
    load_scale_part(k0, p);
  };
  auto load_full = [&](int kt, uint8_t* dA, uint8_t* dB) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 8; ++p) load_part(kt, dA, dB, p);
  };
  auto read_frag = [&](const uint8_t* base, int r, int ks) __attribute__((always_inline)) -> v8i {
    const int c0 = 4 * ks + h, c1 = 4 * ks + 2 + h;
    const int sw = (r >> 1) & 7;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + r * BK + ((c0 ^ sw) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + r * BK + ((c1 ^ sw) << 4));
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  };
  auto take_scales = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) { sb_c[s][0] = sb_n[s][0]; sb_c[s][1] = sb_n[s][1]; }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) { sa_c[mi][0] = sa_n[mi][0]; sa_c[mi][1] = sa_n[mi][1]; }
  };
  // byte-0-aligned scale register of k-step ks: block h (ks 0) or 2+h (ks 1)
  auto scale_of = [&](uint32_t c0, uint32_t c1, int ks) __attribute__((always_inline)) -> int {
    if constexpr (SVEC) return (int)(c0 >> (8 * h + 16 * ks));
    else return (int)(ks == 0 ? c0 : c1);
  };
  // MFMAs of one 128-wide k tile (2 MFMA k-steps x 4 m sub-tiles x 4 n
  // sub-tiles). Fragment reads run one step ahead of the MFMAs that use them:
  // the next A fragment is read under the current m sub-tile's 4 MFMAs, and
  // the B fragments of k-step 1 under the last m sub-tile of k-step 0. Peak
  // fragment registers: 2 x 4 B + 2 A fragments (80 VGPRs).
  auto compute = [&](const uint8_t* sA, const uint8_t* sB, int kt_next, uint8_t* nA, uint8_t* nB)
      __attribute__((always_inline)) {
    v8i fb_c[4], fb_n[4], fa_c, fa_n;
    static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
      constexpr int s = decltype(s_c)::value;
      fb_c[s] = read_frag(sB, nsub(s) + l32, 0);
    });
    fa_c = read_frag(sA, 128 * wm + l32, 0);
    static_for<0, 8>([&](auto step_c) __attribute__((always_inline)) {
      constexpr int step = decltype(step_c)::value;
      constexpr int ks = step / 4, mi = step % 4;
      load_part(kt_next, nA, nB, step);
      if constexpr (step < 7) fa_n = read_frag(sA, 128 * wm + 32 * ((step + 1) % 4) + l32, (step + 1) / 4);
      if constexpr (step == 3) {
        static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          fb_n[s] = read_frag(sB, nsub(s) + l32, 1);
        });
      }
      static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        acc[s][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb_c[s], fa_c, acc[s][mi], 0, 0, 0, scale_of(sb_c[s][0], sb_c[s][1], ks), 0,
            scale_of(sa_c[mi][0], sa_c[mi][1], ks));
      });
      // fence: each step's slice of loads stays with its 4 MFMAs
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (step < 7) fa_c = fa_n;
      if constexpr (step == 3) {
        static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          fb_c[s] = fb_n[s];
        });
      }
    });
  };
  // Zero the chunks of a staged k-step that lie past klen (the k tail of a
  // group-K tile): each lane clears the LDS slots it loaded.
  auto zero_tail = [&](int kt, uint8_t* dA, uint8_t* dB) __attribute__((always_inline)) {
    const bool ok = kt * BK + lch * 16 < klen;
    if (!ok) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int blk = it * 4 + wave;
        *reinterpret_cast<uint4*>(dA + blk * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(dB + blk * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // One k-step: prefetch k-step kt+1 into (nA, nB) interleaved with the MFMAs
  // of stage (cA, cB), wait for this wave's loads, then hand the stages over
  // (barrier). The prefetch is unconditional: past the last k-step it reads
  // bytes the bounds-checked buffer returns as 0 or data of neighbouring rows,
  // into the stage nobody computes on again. A partial last k-step (group-K
  // tail) gets its out-of-range chunks zeroed after the handoff.
  auto kstep = [&](int kt, const uint8_t* cA, const uint8_t* cB, uint8_t* nA, uint8_t* nB)
      __attribute__((always_inline)) {
    compute(cA, cB, kt + 1, nA, nB);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    take_scales();
    __syncthreads();
    if ((klen & (BK - 1)) != 0 && kt + 2 == nk) {
      zero_tail(kt + 1, nA, nB);
      __syncthreads();
    }
  };

  if (nk > 0) {
    load_full(0, sA0, sB0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    take_scales();
    __syncthreads();
    if ((klen & (BK - 1)) != 0 && nk == 1) {
      zero_tail(0, sA0, sB0);
      __syncthreads();
    }
  }
  // k-step kt lives in stage kt & 1
  for (int kt = 0; kt < nk; kt += 2) {
    kstep(kt, sA0, sB0, sA1, sB1);
    if (kt + 1 < nk) kstep(kt + 1, sA1, sB1, sA0, sB0);
  }

  // ---------------------------------------------------------------- epilogues
  // lane holds, for n sub-tile s and m sub-tile mi: m_local = 128*wm + 32*mi + l32,
  // n_local = nsub(s) + 8*(v/4) + 4*h + (v%4) for v = 0..15.
  // The per-lane indices are re-derived from an opaque copy of the lane id so
  // that no epilogue address is computed before (and kept live across) the
  // main loop.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  {
  const int h = lane_e >> 5;        // shadows of the loop's lane-derived values
  const int l32 = lane_e & 31;
  const int tid = wave * 64 + lane_e;
  if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
    if (MODE == MX_GROUP_K && klen == 0 && args.accumulate) return;
    // Direct stores: per instruction, lanes (l, l^32) write 8 consecutive
    // columns of 32 rows; the 4 column groups of a sub-tile complete each
    // row's 128-byte (fp32) or 64-byte (bf16) run, which L2 merges.
    char* cbase = reinterpret_cast<char*>(args.c);
    constexpr int esz = EPI == EPI_F32 ? 4 : 2;
    if constexpr (MODE == MX_GROUP_K) cbase += (int64_t)g * args.c_group_stride * esz;
    // accumulate and overwrite are separate code paths so the accumulator
    // registers never merge with the loaded old values
    auto store_tile = [&](auto acc_c) __attribute__((always_inline)) {
      constexpr bool ACC = decltype(acc_c)::value;
      static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
        constexpr int mi = decltype(mi_c)::value;
        const int ml = 128 * wm + 32 * mi + l32;
        const bool row_ok = ml < a_rows_valid;
        const int64_t m = a_row0 + ml;
        static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          __builtin_amdgcn_sched_barrier(0);
          const int64_t n0 = (int64_t)tc.nt * BN + nsub(s) + 4 * h;
          if (row_ok && n0 < args.N) {
            char* rowp = cbase + (m * args.ldc + n0) * esz;
            static_for<0, 4>([&](auto vg_c) __attribute__((always_inline)) {
              constexpr int vg = decltype(vg_c)::value;
              float c0 = acc[s][mi][4 * vg + 0], c1 = acc[s][mi][4 * vg + 1];
              float c2 = acc[s][mi][4 * vg + 2], c3 = acc[s][mi][4 * vg + 3];
              if constexpr (EPI == EPI_F32) {
                c0 = vgpr_hop(c0); c1 = vgpr_hop(c1); c2 = vgpr_hop(c2); c3 = vgpr_hop(c3);
                float4* p = reinterpret_cast<float4*>(rowp + 8 * vg * 4);
                if constexpr (ACC) {
                  const float4 old = *p;
                  c0 += old.x; c1 += old.y; c2 += old.z; c3 += old.w;
                }
                *p = make_float4(c0, c1, c2, c3);
              } else {
                uint2 o;
                o.x = pack_bf16x2(c0, c1);
                o.y = pack_bf16x2(c2, c3);
                *reinterpret_cast<uint2*>(rowp + 8 * vg * 2) = o;
              }
            });
          }
        });
      });
    };
    if (EPI == EPI_F32 && args.accumulate) store_tile(std::true_type{});
    else store_tile(std::false_type{});
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    // sub-tiles s (gate) and s+2 (up), s = 0,1, cover ffn columns
    // j = j0(s) + 8*(v/4) + 4*h + v%4 with j0(s) = nt*128 + 64*wn + 32*s.
    const int F = args.F;
    const int64_t pc0 = args.groups.pc0[slot];
    const int64_t ldc = args.ld_col;
    const int grow_in_group0 = tc.mt * BM;
    static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
      constexpr int mi = decltype(mi_c)::value;
      const int ml = 128 * wm + 32 * mi + l32;
      const bool row_ok = ml < a_rows_valid;
      const int64_t m = a_row0 + ml;
      __builtin_amdgcn_sched_barrier(0);
      const float w = row_ok ? (args.probs ? args.probs[m] : 1.0f) : 0.0f;
      const int blk_row = grow_in_group0 + 128 * wm + 32 * mi;  // first row of the 32-row block in the group
      const bool blk_in_layout = blk_row < args.groups.len[slot];
      static_for<0, 2>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int j0 = tc.nt * (BN / 2) + 64 * wn + 32 * s;
        const bool jblk_ok = j0 < F;           // F % 32 == 0: whole 32-block valid or not
        float a[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float gg = vgpr_hop(acc[s][mi][v]), uu = vgpr_hop(acc[s + 2][mi][v]);
          const float sl = gg / (1.0f + __expf(-gg));
          a[v] = row_ok ? w * sl * uu : 0.0f;
        }
        if (args.h1 != nullptr && row_ok && jblk_ok) {
#pragma unroll
          for (int vg = 0; vg < 4; ++vg) {
            const int64_t j = j0 + 8 * vg + 4 * h;
            uint2 og, ou;
            og.x = pack_bf16x2(acc[s][mi][4 * vg], acc[s][mi][4 * vg + 1]);
            og.y = pack_bf16x2(acc[s][mi][4 * vg + 2], acc[s][mi][4 * vg + 3]);
            ou.x = pack_bf16x2(acc[s + 2][mi][4 * vg], acc[s + 2][mi][4 * vg + 1]);
            ou.y = pack_bf16x2(acc[s + 2][mi][4 * vg + 2], acc[s + 2][mi][4 * vg + 3]);
            *reinterpret_cast<uint2*>(args.h1 + m * 2 * F + j) = og;
            *reinterpret_cast<uint2*>(args.h1 + m * 2 * F + F + j) = ou;
          }
        }
        // rowwise MXFP8 of A: block = the 32 j's of this sub-tile (lanes l, l^32)
        {
          uint32_t am = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) am = umax(am, abs_bits(a[v]));
          am = umax(am, xor_u32(am, 32));
          const uint32_t sc = scale_code_from_amax_bits(am);
          const float inv = inv_scale_from_code(sc);
          if (row_ok && jblk_ok) {
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
              const uint32_t q = e4m3x4(a[4 * vg] * inv, a[4 * vg + 1] * inv, a[4 * vg + 2] * inv, a[4 * vg + 3] * inv);
              *reinterpret_cast<uint32_t*>(args.q_row + m * F + j0 + 8 * vg + 4 * h) = q;
            }
            if (h == 0) args.s_row[m * (F / 32) + j0 / 32] = (uint8_t)sc;
          }
        }
        // columnwise MXFP8 of A: block = the 32 rows of this m sub-tile (one lane half)
        if (args.q_col != nullptr && blk_in_layout && jblk_ok) {
          static_for<0, 16>([&](auto v_c) __attribute__((always_inline)) {
            constexpr int v = decltype(v_c)::value;
            uint32_t am = abs_bits(a[v]);
            static_for<0, 5>([&](auto k_c) __attribute__((always_inline)) {
              am = umax(am, xor_u32(am, 1 << decltype(k_c)::value));
            });
            const uint32_t sc = scale_code_from_amax_bits(am);
            const float inv = inv_scale_from_code(sc);
            const uint32_t q = e4m3x4(a[v] * inv, 0.0f, 0.0f, 0.0f) & 0xFFu;
            const int64_t j = j0 + 8 * (v >> 2) + 4 * h + (v & 3);
            args.q_col[j * ldc + pc0 + blk_row + l32] = (uint8_t)q;
            if (l32 == 0) args.s_col[j * (ldc / 32) + (pc0 + blk_row) / 32] = (uint8_t)sc;
          });
        }
      });
    });
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dA for ffn column j = nt*256 + nsub(s) + 8*(v/4) + 4*h + v%4
    const int F = args.F;
    const int64_t pc0 = args.groups.pc0[slot];
    const int64_t ldc = args.ld_col;
    const int grow_in_group0 = tc.mt * BM;
    float dpsum[4];
    static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
      constexpr int mi = decltype(mi_c)::value;
      const int ml = 128 * wm + 32 * mi + l32;
      const bool row_ok = ml < a_rows_valid;
      const int64_t m = a_row0 + ml;
      __builtin_amdgcn_sched_barrier(0);
      const float w = row_ok ? (args.probs ? args.probs[m] : 1.0f) : 0.0f;
      const int blk_row = grow_in_group0 + 128 * wm + 32 * mi;
      const bool blk_in_layout = blk_row < args.groups.len[slot];
      float dp = 0.0f;
      static_for<0, 4>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int j0 = tc.nt * BN + nsub(s);
        const bool jblk_ok = j0 < F;
        float dg[16], du[16];
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int64_t j = j0 + 8 * vg + 4 * h;
          uint2 gr = make_uint2(0, 0), ur = make_uint2(0, 0);
          if (row_ok && jblk_ok) {
            gr = *reinterpret_cast<const uint2*>(args.h1 + m * 2 * F + j);
            ur = *reinterpret_cast<const uint2*>(args.h1 + m * 2 * F + F + j);
          }
          const float gv[4] = {bf16_lo(gr.x), bf16_hi(gr.x), bf16_lo(gr.y), bf16_hi(gr.y)};
          const float uv[4] = {bf16_lo(ur.x), bf16_hi(ur.x), bf16_lo(ur.y), bf16_hi(ur.y)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float da = vgpr_hop(acc[s][mi][4 * vg + i]);
            const float sg = 1.0f / (1.0f + __expf(-gv[i]));
            const float sl = gv[i] * sg;
            const float dgv = da * w * uv[i] * sg * (1.0f + gv[i] * (1.0f - sg));
            const float duv = da * w * sl;
            const bool ok = row_ok && jblk_ok;
            dg[4 * vg + i] = ok ? dgv : 0.0f;
            du[4 * vg + i] = ok ? duv : 0.0f;
            dp += ok ? da * sl * uv[i] : 0.0f;
          }
        }
        // MXFP8 of dg (dH1 columns j) and du (dH1 columns F + j), both layouts
        static_for<0, 2>([&](auto half_c) __attribute__((always_inline)) {
          constexpr int half = decltype(half_c)::value;
          float d[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) d[v] = half == 0 ? dg[v] : du[v];
          const int64_t jc0 = (half == 0 ? 0 : (int64_t)F) + j0;
          __builtin_amdgcn_sched_barrier(0);
          uint32_t am = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) am = umax(am, abs_bits(d[v]));
          am = umax(am, xor_u32(am, 32));
          const uint32_t sc = scale_code_from_amax_bits(am);
          const float inv = inv_scale_from_code(sc);
          if (row_ok && jblk_ok) {
#pragma unroll
            for (int vg = 0; vg < 4; ++vg) {
              const uint32_t q = e4m3x4(d[4 * vg] * inv, d[4 * vg + 1] * inv, d[4 * vg + 2] * inv, d[4 * vg + 3] * inv);
              *reinterpret_cast<uint32_t*>(args.q_row + m * 2 * F + jc0 + 8 * vg + 4 * h) = q;
            }
            if (h == 0) args.s_row[m * (2 * F / 32) + jc0 / 32] = (uint8_t)sc;
          }
          if (blk_in_layout && jblk_ok) {
            static_for<0, 16>([&](auto v_c) __attribute__((always_inline)) {
              constexpr int v = decltype(v_c)::value;
              uint32_t amc = abs_bits(d[v]);
              static_for<0, 5>([&](auto k_c) __attribute__((always_inline)) {
                amc = umax(amc, xor_u32(amc, 1 << decltype(k_c)::value));
              });
              const uint32_t scc = scale_code_from_amax_bits(amc);
              const float invc = inv_scale_from_code(scc);
              const uint32_t q = e4m3x4(d[v] * invc, 0.0f, 0.0f, 0.0f) & 0xFFu;
              const int64_t jc = jc0 + 8 * (v >> 2) + 4 * h + (v & 3);
              args.q_col[jc * ldc + pc0 + blk_row + l32] = (uint8_t)q;
              if (l32 == 0) args.s_col[jc * (ldc / 32) + (pc0 + blk_row) / 32] = (uint8_t)scc;
            });
          }
        });
      });
      dp += xor_f32(dp, 32);
      dpsum[mi] = dp;
    });
    // dprobs partial over this tile's 256 columns: reduce the 2 n-waves via LDS
    if (args.dprobs_part != nullptr) {
      float* red = reinterpret_cast<float*>(sA0);   // main loop is done (barrier above)
      if (h == 0) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) red[wn * BM + 128 * wm + 32 * mi + l32] = dpsum[mi];
      }
      __syncthreads();
      if (tid < a_rows_valid) {
        const float tot = red[tid] + red[BM + tid];
        args.dprobs_part[(int64_t)tc.nt * args.R + a_row0 + tid] = tot;
      }
    }
  }
  }  // epilogue scope
#endif  // __HIP_DEVICE_COMPILE__
}

__global__ __launch_bounds__(256) void dprobs_reduce_kernel(const float* part, float* out, int32_t R, int32_t n_parts) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  float s = 0.0f;
  for (int p = 0; p < n_parts; ++p) s += part[(int64_t)p * R + r];
  out[r] = s;
}

template <int MODE, int EPI>
static hipError_t launch_mode_epi(bool svec, const GemmArgs& args, int total, hipStream_t stream) {
  if (svec)
    hipLaunchKernelGGL((gemm_kernel<MODE, EPI, true>), dim3(total), dim3(kThreads), 0, stream, args, total);
  else
    hipLaunchKernelGGL((gemm_kernel<MODE, EPI, false>), dim3(total), dim3(kThreads), 0, stream, args, total);
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, int epi, bool scale_dword, const GemmArgs& args, int total_tiles,
                       hipStream_t stream) {
  if (total_tiles == 0) return hipSuccess;
  if (mode == MX_GROUP_M) {
    switch (epi) {
      case EPI_F32: return launch_mode_epi<MX_GROUP_M, EPI_F32>(scale_dword, args, total_tiles, stream);
      case EPI_BF16: return launch_mode_epi<MX_GROUP_M, EPI_BF16>(scale_dword, args, total_tiles, stream);
      case EPI_SWIGLU_FWD: return launch_mode_epi<MX_GROUP_M, EPI_SWIGLU_FWD>(scale_dword, args, total_tiles, stream);
      case EPI_SWIGLU_BWD: return launch_mode_epi<MX_GROUP_M, EPI_SWIGLU_BWD>(scale_dword, args, total_tiles, stream);
    }
  } else {
    switch (epi) {
      case EPI_F32: return launch_mode_epi<MX_GROUP_K, EPI_F32>(false, args, total_tiles, stream);
      case EPI_BF16: return launch_mode_epi<MX_GROUP_K, EPI_BF16>(false, args, total_tiles, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dprobs_reduce(const float* part, float* dprobs, int32_t R, int32_t n_parts, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(dprobs_reduce_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, part, dprobs, R, n_parts);
  return hipGetLastError();
}

}  // namespace mx
