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
// row r stored at chunk (c ^ (r & 7)) so that the 8 rows read together by one
// ds_read_b128 phase hit distinct banks. Global loads go through registers
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

// Scale bytes of one row for the two MFMA k-steps of a 128-wide k tile:
// returns byte-0-aligned registers for k-step 0 (block h) and 1 (block 2+h).
template <bool SVEC>
__device__ __forceinline__ void load_scale_pair(const uint8_t* srow, int blk0, int blk_last, int h,
                                                uint32_t& s0, uint32_t& s1) {
  if constexpr (SVEC) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(srow + blk0);
    s0 = w >> (8 * h);
    s1 = w >> (8 * h + 16);
  } else {
    int b0 = min(blk0 + h, blk_last);
    int b1 = min(blk0 + 2 + h, blk_last);
    s0 = srow[b0];
    s1 = srow[b1];
  }
}

template <int MODE, int EPI, bool SVEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs args, int total_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][BM * BK];   // [buf][A/B][row*128]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  if (a_rows_valid > BM) a_rows_valid = BM;
  const int nk = (klen + BK - 1) / BK;
  const int64_t lds_a = args.lda / 32, lds_b = args.ldb / 32;
  const int blk_last = (int)((kbeg + klen) / 32) - 1;  // last valid k block (clamp target)
  const uint8_t* a_base = args.a + a_row0 * args.lda + kbeg;
  const uint8_t* as_base = args.as + a_row0 * lds_a;

  // tile-local B row r -> row of B_g (SwiGLU fwd: gate/up pairing); clamped in-bounds
  auto b_row_of = [&](int r) -> uint32_t {
    if constexpr (EPI == EPI_SWIGLU_FWD) {
      const int j = tc.nt * (BN / 2) + (r & (BN / 2 - 1));
      const int jc = j < args.F ? j : args.F - 1;
      return (uint32_t)((r < BN / 2) ? jc : args.F + jc);
    } else {
      const int n = tc.nt * BN + r;
      return (uint32_t)(n < args.N ? n : args.N - 1);
    }
  };
  auto a_row_of = [&](int r) -> uint32_t { return (uint32_t)(r < a_rows_valid ? r : a_rows_valid - 1); };
  auto nsub = [&](int s) -> int { return (s < 2 ? 64 * wn + 32 * s : BN / 2 + 64 * wn + 32 * (s - 2)); };

  // ---- direct global->LDS loads: per k-step each wave fills 8 blocks of 1 KB
  // (8 tile rows) of A and of B; LDS slot = lane, i.e. row 8*blk + lane/8 and
  // stored chunk lane%8, which holds logical chunk (lane%8) ^ (lane/8).
  uint32_t a_off[8], b_off[8];
  const int lch = (lane & 7) ^ (lane >> 3);   // logical 16-byte chunk this lane fetches
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = 8 * (it * 4 + wave) + (lane >> 3);
    a_off[it] = a_row_of(r) * (uint32_t)args.lda + lch * 16;
    b_off[it] = b_row_of(r) * (uint32_t)args.ldb + lch * 16;
  }
  const uint8_t* b_base = bq + kbeg;

  // ---- per-lane scale rows: B sub-tiles s = 0..3 and A sub-tiles mi = 0..3
  uint32_t bs_off[4], as_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) bs_off[s] = b_row_of(nsub(s) + l32) * (uint32_t)lds_b;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) as_off[mi] = a_row_of(128 * wm + 32 * mi + l32) * (uint32_t)lds_a;

  v16f acc[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][mi][v] = 0.0f;

  uint32_t sb_n[4][2], sa_n[4][2];   // prefetched scales (next k-step)
  uint32_t sb_c[4][2], sa_c[4][2];   // current

  // issue the loads of k-step kt into LDS buffer buf (and its scales into registers)
  auto global_load = [&](int kt, int buf) {
    const int k0 = kt * BK;
    const bool ok = k0 + lch * 16 < klen;
    const uint8_t* ab = a_base + k0;
    const uint8_t* bb = b_base + k0;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      uint8_t* da = &smem[buf][0][(it * 4 + wave) * 1024];
      uint8_t* db = &smem[buf][1][(it * 4 + wave) * 1024];
      if (ok) {
        __builtin_amdgcn_global_load_lds(ab + a_off[it], (__attribute__((address_space(3))) void*)da, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(bb + b_off[it], (__attribute__((address_space(3))) void*)db, 16, 0, 0);
      } else {
        *reinterpret_cast<uint4*>(da + lane * 16) = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(db + lane * 16) = make_uint4(0, 0, 0, 0);
      }
    }
    const int blk0 = (int)((kbeg + k0) / 32);
#pragma unroll
    for (int s = 0; s < 4; ++s) load_scale_pair<SVEC>(bsc + bs_off[s], blk0, blk_last, h, sb_n[s][0], sb_n[s][1]);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) load_scale_pair<SVEC>(as_base + as_off[mi], blk0, blk_last, h, sa_n[mi][0], sa_n[mi][1]);
  };
  auto read_frag = [&](const uint8_t* base, int r, int ks) -> v8i {
    const int c0 = 4 * ks + h, c1 = 4 * ks + 2 + h;
    const uint4 lo = *reinterpret_cast<const uint4*>(base + r * BK + ((c0 ^ (r & 7)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(base + r * BK + ((c1 ^ (r & 7)) << 4));
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
  };

  if (nk > 0) {
    global_load(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < 4; ++s) { sb_c[s][0] = sb_n[s][0]; sb_c[s][1] = sb_n[s][1]; }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) { sa_c[mi][0] = sa_n[mi][0]; sa_c[mi][1] = sa_n[mi][1]; }
    __syncthreads();
  }

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) global_load(kt + 1, buf ^ 1);
    const uint8_t* sA = smem[buf][0];
    const uint8_t* sB = smem[buf][1];
    static_for<0, 2>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      v8i fb[4];
      static_for<0, 4>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        fb[s] = read_frag(sB, nsub(s) + l32, ks);
      });
      static_for<0, 4>([&](auto mi_c) {
        constexpr int mi = decltype(mi_c)::value;
        const v8i fa = read_frag(sA, 128 * wm + 32 * mi + l32, ks);
        static_for<0, 4>([&](auto s_c) {
          constexpr int s = decltype(s_c)::value;
          acc[s][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fb[s], fa, acc[s][mi], 0, 0, 0, (int)sb_c[s][ks], 0, (int)sa_c[mi][ks]);
        });
      });
    });
    if (more) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int s = 0; s < 4; ++s) { sb_c[s][0] = sb_n[s][0]; sb_c[s][1] = sb_n[s][1]; }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) { sa_c[mi][0] = sa_n[mi][0]; sa_c[mi][1] = sa_n[mi][1]; }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogues
  // lane holds, for n sub-tile s and m sub-tile mi: m_local = 128*wm + 32*mi + l32,
  // n_local = nsub(s) + 8*(v/4) + 4*h + (v%4) for v = 0..15.
  if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
    if (MODE == MX_GROUP_K && klen == 0 && args.accumulate) return;
    char* cbase = reinterpret_cast<char*>(args.c);
    const int esz = EPI == EPI_F32 ? 4 : 2;
    if constexpr (MODE == MX_GROUP_K) cbase += (int64_t)g * args.c_group_stride * esz;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int ml = 128 * wm + 32 * mi + l32;
      if (ml >= a_rows_valid) continue;
      const int64_t m = a_row0 + ml;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int64_t n = (int64_t)tc.nt * BN + nsub(s) + 8 * vg + 4 * h;
          if (n >= args.N) continue;
          const float c0 = acc[s][mi][4 * vg + 0], c1 = acc[s][mi][4 * vg + 1];
          const float c2 = acc[s][mi][4 * vg + 2], c3 = acc[s][mi][4 * vg + 3];
          if constexpr (EPI == EPI_F32) {
            float4* p = reinterpret_cast<float4*>(cbase + (m * args.ldc + n) * 4);
            float4 o = make_float4(c0, c1, c2, c3);
            if (args.accumulate) {
              const float4 old = *p;
              o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
            }
            *p = o;
          } else {
            uint2 o;
            o.x = pack_bf16x2(c0, c1);
            o.y = pack_bf16x2(c2, c3);
            *reinterpret_cast<uint2*>(cbase + (m * args.ldc + n) * 2) = o;
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    // sub-tiles s (gate) and s+2 (up), s = 0,1, cover ffn columns
    // j = j0(s) + 8*(v/4) + 4*h + v%4 with j0(s) = nt*128 + 64*wn + 32*s.
    const int F = args.F;
    const int64_t pc0 = args.groups.pc0[slot];
    const int64_t ldc = args.ld_col;
    const int grow_in_group0 = tc.mt * BM;
    static_for<0, 4>([&](auto mi_c) {
      constexpr int mi = decltype(mi_c)::value;
      const int ml = 128 * wm + 32 * mi + l32;
      const bool row_ok = ml < a_rows_valid;
      const int64_t m = a_row0 + ml;
      __builtin_amdgcn_sched_barrier(0);
      const float w = row_ok ? (args.probs ? args.probs[m] : 1.0f) : 0.0f;
      const int blk_row = grow_in_group0 + 128 * wm + 32 * mi;  // first row of the 32-row block in the group
      const bool blk_in_layout = blk_row < args.groups.len[slot];
      static_for<0, 2>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        const int j0 = tc.nt * (BN / 2) + 64 * wn + 32 * s;
        const bool jblk_ok = j0 < F;           // F % 32 == 0: whole 32-block valid or not
        float a[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float gg = acc[s][mi][v], uu = acc[s + 2][mi][v];
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
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            uint32_t am = abs_bits(a[v]);
#pragma unroll
            for (int sh = 1; sh < 32; sh <<= 1) am = umax(am, xor_u32(am, sh));
            const uint32_t sc = scale_code_from_amax_bits(am);
            const float inv = inv_scale_from_code(sc);
            const uint32_t q = e4m3x4(a[v] * inv, 0.0f, 0.0f, 0.0f) & 0xFFu;
            const int64_t j = j0 + 8 * (v >> 2) + 4 * h + (v & 3);
            args.q_col[j * ldc + pc0 + blk_row + l32] = (uint8_t)q;
            if (l32 == 0) args.s_col[j * (ldc / 32) + (pc0 + blk_row) / 32] = (uint8_t)sc;
          }
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
    static_for<0, 4>([&](auto mi_c) {
      constexpr int mi = decltype(mi_c)::value;
      const int ml = 128 * wm + 32 * mi + l32;
      const bool row_ok = ml < a_rows_valid;
      const int64_t m = a_row0 + ml;
      __builtin_amdgcn_sched_barrier(0);
      const float w = row_ok ? (args.probs ? args.probs[m] : 1.0f) : 0.0f;
      const int blk_row = grow_in_group0 + 128 * wm + 32 * mi;
      const bool blk_in_layout = blk_row < args.groups.len[slot];
      float dp = 0.0f;
      static_for<0, 4>([&](auto s_c) {
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
            const float da = acc[s][mi][4 * vg + i];
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
        auto quant_out = [&](const float (&d)[16], int64_t jc0) {
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
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              uint32_t amc = abs_bits(d[v]);
#pragma unroll
              for (int sh = 1; sh < 32; sh <<= 1) amc = umax(amc, xor_u32(amc, sh));
              const uint32_t scc = scale_code_from_amax_bits(amc);
              const float invc = inv_scale_from_code(scc);
              const uint32_t q = e4m3x4(d[v] * invc, 0.0f, 0.0f, 0.0f) & 0xFFu;
              const int64_t jc = jc0 + 8 * (v >> 2) + 4 * h + (v & 3);
              args.q_col[jc * ldc + pc0 + blk_row + l32] = (uint8_t)q;
              if (l32 == 0) args.s_col[jc * (ldc / 32) + (pc0 + blk_row) / 32] = (uint8_t)scc;
            }
          }
        };
        quant_out(dg, j0);
        __builtin_amdgcn_sched_barrier(0);
        quant_out(du, (int64_t)F + j0);
      });
      dp += xor_f32(dp, 32);
      dpsum[mi] = dp;
    });
    // dprobs partial over this tile's 256 columns: reduce the 2 n-waves via LDS
    if (args.dprobs_part != nullptr) {
      float* red = reinterpret_cast<float*>(&smem[0][0][0]);   // main loop is done (barrier above)
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
