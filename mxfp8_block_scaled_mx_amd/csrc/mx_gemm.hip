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
// and four 32-row n sub-tiles: n [128*wn, +128) for the plain epilogues, and
// {64*wn, 64*wn+32, 128+64*wn, 160+64*wn} with the SwiGLU pairing (tile rows
// 0..127 = gate rows, 128..255 = the matching up rows), so that sub-tiles s
// and s+2 hold gate and up of the same (row, j) in the same accumulator slot.
// The MFMA's first operand is the B tile (n), its second the A tile (m), so
// each lane ends up with one m row (lane % 32) and 16 n values: 4 runs of 4
// consecutive n, the 32 n of one MXFP8 block in lanes l and l^32.
//
// Operand layout inside the MFMA (pinned on hardware): lane l = row (l%32),
// half h = l/32 holds k [16h, 16h+16) in bytes 0-15 and k [32+16h, +16) in
// bytes 16-31 of its 32-byte operand; the scale register of lane l (byte 0)
// scales k-block h of its row.
//
// Operands: double-buffered A and B stages in LDS, filled straight from
// global memory by buffer->LDS DMA one k-step ahead, 128 bytes per row with
// 16-byte chunk c of row r stored at chunk (c ^ ((r >> 1) & 7)), so that
// fragment reads are free of bank conflicts. Each wave also touches the L2
// lines of its share of the operand rows three k-steps ahead. Scales come
// per lane from global memory (row layouts) or, for the k-tiled layout of
// the fused MLP, by DMA into a small LDS stage beside the operands.
//
// Tile order: workgroup ids are spread over the 8 XCDs in rounds of 32
// consecutive tile ids per XCD (the tiles one XCD runs together share A and
// B rows in its L2), then mapped to (group, m-tile, n-tile) with m-tiles in
// bands of 8. Plain group-M GEMMs split the tiles of a last, partial round
// along k (fp32 partials, summed by split_reduce_kernel).
//
// Epilogues: fp32 (optionally accumulating) and bf16 C; the fused SwiGLU
// forward (A = w * silu(g) * u, H1 saved as bf16, A quantized rowwise and
// columnwise) and backward (dg, du, dprobs partials, dH1 quantized rowwise
// and columnwise). fp32 C leaves through LDS as whole 128-byte rows.
#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

[[maybe_unused]] constexpr int BM = kTileM, BN = kTileN, BK = kTileK;
static_assert(sizeof(GemmArgs) <= 4096, "kernel arguments must fit the 4 KB kernarg segment");
// Waves: 2 along m (128 rows each) x kWavesN along n. kWavesN = 2: a wave
// owns 128 x 128 (NS = 4 n sub-tiles of 32, 256 fp32 accumulators in AGPRs),
// one wave per SIMD. (kWavesN = 4 -- 128 x 64 per wave, two waves per SIMD --
// is also supported, but at 256 registers per wave the accumulators leave the
// AGPRs and the loop spills, which makes it slower.)
constexpr int kWavesN = 2;
constexpr int kWaves = 2 * kWavesN;
constexpr int kThreads = 64 * kWaves;
[[maybe_unused]] constexpr int NS = 8 / kWavesN;   // n sub-tiles of 32 per wave
[[maybe_unused]] constexpr int kWaveN = 256 / kWavesN;      // n columns per wave
[[maybe_unused]] constexpr int kDmaPerWave = 32 / kWaves;    // 1 KB blocks of A (and of B) per wave per k-step
// m-tiles per band of the raster: 8 for group-M (fprop, dgrad); 4 for
// group-K (wgrad), measured faster there (wgrad1 of the Mixtral-shaped
// backward 1.99 -> 1.90 ms) while slower for group-M
__host__ __device__ constexpr int band_m(int mode) { return mode == MX_GROUP_K ? 4 : 8; }
// L2 prefetch distance in k-steps (see kstep)
[[maybe_unused]] constexpr int kPrefetchAhead = 3;
// Epilogue transpose area of a 32 x 32 fp32 block in a wave's LDS slice:
// [column][row] with 36 floats per column (a multiple of 4 for the 16-byte
// reads; the 8 lanes of one 16-byte read pass start 4 banks apart)
[[maybe_unused]] constexpr int kTrStride = 36;
[[maybe_unused]] constexpr int kTrBytes = 32 * kTrStride * 4;
// cache policy of memory touched exactly once (fp32 C of the plain epilogue):
// non-temporal
[[maybe_unused]] constexpr int kNonTemporal = 2;

struct TileCoord {
  int slot;   // group slot in the table
  int mt, nt; // tile indices within the group
};

// words of k-tiled scales per LDS stage: A 16 row groups, B 8 row groups
[[maybe_unused]] constexpr int kScStage = 768;

// Slot of a tile id: slots hold consecutive id ranges (tile0), except in an
// interleaved group-K plan, where chunk q of kXcdChunk ids belongs to slot
// (q % n + q / n) % n as its chunk q / n. Every n consecutive chunks then
// cover all slots once, so the tiles running at one time mix contractions of
// different lengths (their k-loops and their fp32 read-modify-write phases
// overlap across CUs instead of all CUs computing, then all CUs storing), and
// the rotation gives every XCD the same mix, while the 32 tiles one XCD runs
// together still come from one slot and share its operand rows in L2.
__device__ __forceinline__ TileCoord locate_tile(const GemmGroups& gt, int id, int mode, int M, int n_tiles_n) {
  int lo = 0, local;
  if (mode == MX_GROUP_K && gt.interleave) {
    const int q = id / kXcdChunk, r = q / gt.n, pos = q - r * gt.n;
    lo = pos + r % gt.n;
    if (lo >= gt.n) lo -= gt.n;
    local = r * kXcdChunk + (id - q * kXcdChunk);
  } else {
    int hi = gt.n - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (gt.tile0[mid] <= id) lo = mid; else hi = mid - 1;
    }
    local = id - gt.tile0[lo];
  }
  TileCoord t;
  t.slot = lo;
  const int rows = mode == MX_GROUP_M ? gt.len[lo] : M;
  const int mtiles = (rows + BM - 1) / BM;
  // band raster: band_m(mode) m-tiles x all n-tiles, m fastest inside a band
  const int kBandM = band_m(mode);
  const int per_band = kBandM * n_tiles_n;
  const int band = local / per_band;
  const int in_band = local - band * per_band;
  const int band_m0 = band * kBandM;
  const int band_h = min(kBandM, mtiles - band_m0);
  t.mt = band_m0 + in_band % band_h;
  t.nt = in_band / band_h;
  return t;
}

// Scale sources: per-lane byte loads (any layout), per-lane dword loads (row
// layouts whose 4 scales of a k-step are one aligned word), or the k-tiled
// layout through LDS (one DMA per 256 rows and k-step).
enum ScaleSource : int { kScByte = 0, kScDword = 1, kScLds = 2 };

template <bool DEVG>
__device__ __forceinline__ const GemmGroups& gemm_groups(const GemmArgs& a) {
  if constexpr (DEVG) return *a.groups_dev;
  else return a.groups;
}

// DEVG: the group table is in device memory (args.groups_dev), built there
// from device-resident group sizes; the grid is sized for the worst case and
// the workgroups past the table's tile count exit at once.
template <int MODE, int EPI, int SC, bool DEVG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
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
  // k-tiled scales of the two stages: A words of 16 row groups (the tile's 256
  // rows from the group of its first row on) and B words of 8 row groups
  __shared__ __attribute__((aligned(16))) uint32_t sSc[SC == kScLds ? 2 * kScStage : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Work unit of this workgroup: a whole tile, or (split-K tail) part
  // `part` of tile id's k-steps, written as an fp32 partial tile.
  const GemmGroups& gt = gemm_groups<DEVG>(args);
  if constexpr (DEVG) {
    total_tiles = gt.tile0[gt.n];
    if ((int)blockIdx.x >= total_tiles) return;
  }
  int id, part = 0, split_unit = -1;
  if (!DEVG && args.split_s > 1 && (int)blockIdx.x >= args.split_f) {
    split_unit = (int)blockIdx.x - args.split_f;
    id = args.split_f + split_unit / args.split_s;
    part = split_unit % args.split_s;
  } else {
    id = xcd_remap(blockIdx.x, args.split_s > 1 ? args.split_f : total_tiles);
  }
  const TileCoord tc = locate_tile(gt, id, MODE, args.M, args.n_tiles_n);
  const int slot = tc.slot;
  const int g = gt.gid[slot];

  // ---- geometry of this tile
  int64_t a_row0;     // first global A row of the tile
  int a_rows_valid;   // rows of A valid in this tile (from a_row0)
  int64_t kbeg;       // first k column
  int klen;           // k columns to contract (multiple of 32)
  int b_rows;         // rows of B_g
  const uint8_t* bq = args.b;
  const uint8_t* bsc = args.bs;
  if constexpr (MODE == MX_GROUP_M) {
    a_row0 = (int64_t)gt.a0[slot] + (int64_t)tc.mt * BM;
    a_rows_valid = gt.len[slot] - tc.mt * BM;
    kbeg = 0;
    klen = args.K;
    bq += (int64_t)g * args.b_group_stride;
    bsc += (int64_t)g * args.bs_group_stride;
  } else {
    a_row0 = (int64_t)tc.mt * BM;
    a_rows_valid = args.M - tc.mt * BM;
    kbeg = gt.a0[slot];
    klen = gt.len[slot];
  }
  b_rows = EPI == EPI_SWIGLU_FWD ? 2 * args.F : args.N;
  if (a_rows_valid > BM) a_rows_valid = BM;
  const int nk_all = (klen + BK - 1) / BK;
  // k-steps [kt_lo, kt_hi) of this work unit
  const int kt_lo = split_unit >= 0 ? part * nk_all / args.split_s : 0;
  const int kt_hi = split_unit >= 0 ? (part + 1) * nk_all / args.split_s : nk_all;
  const uint32_t lda = (uint32_t)args.lda, ldb = (uint32_t)args.ldb;
  const int blk_last = (int)((kbeg + klen) / 32) - 1;  // last valid k block (clamp target)
  const ScaleStrides sa = args.sa, sb = args.sb;

  // Operand tiles through buffer resources: rows past the valid ones read as 0.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(args.a + a_row0 * lda + kbeg, (int64_t)(a_rows_valid - 1) * lda + klen);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bq + kbeg, (int64_t)(b_rows - 1) * ldb + klen);
  // Scales: A from the 32-row group of the tile's first row on (rows past the
  // array read 0); B over the rows of B_g, and never past the end of the
  // scale array: in the k-tiled columnwise weight layout the groups sit side
  // by side along k, so B_g's base is g * bs_group_stride into the array
  // while its rows span the array's full row pitch, and the k-step loaded
  // past the last one would otherwise reach beyond the array's last byte.
  const int64_t a_grp0 = (a_row0 >> 5) * sa.grp;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(args.as + a_grp0, args.as_bytes - a_grp0);
  const __amdgpu_buffer_rsrc_t rsb =
      make_rsrc(bsc, MODE == MX_GROUP_M ? min((int64_t)(b_rows >> 5) * sb.grp,
                                              args.bs_bytes - (int64_t)g * args.bs_group_stride)
                                        : args.bs_bytes);

  // first B row of tile row block r0 (a multiple of 8 rows): SwiGLU fwd pairs
  // gate rows [nt*128, +128) (tile rows 0..127) with up rows F + the same j
  auto b_row_base = [&](int r0) __attribute__((always_inline)) -> uint32_t {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      return (uint32_t)((r0 < BN / 2) ? tc.nt * (BN / 2) + r0 : args.F + tc.nt * (BN / 2) + (r0 - BN / 2));
    else
      return (uint32_t)(tc.nt * BN + r0);
  };
  // n sub-tile s of this wave: with the SwiGLU pairing s and s + NS/2 are
  // the gate and up rows of the same 32 ffn columns; otherwise the wave's NS
  // sub-tiles are kWaveN contiguous columns.
  auto nsub = [&](int s) __attribute__((always_inline)) -> int {
    if constexpr (EPI == EPI_SWIGLU_FWD)
      return s < NS / 2 ? (NS / 2) * 32 * wn + 32 * s : BN / 2 + (NS / 2) * 32 * wn + 32 * (s - NS / 2);
    else return kWaveN * wn + 32 * s;
  };

  // ---- direct buffer->LDS loads: per k-step each wave fills kDmaPerWave
  // blocks of 1 KB (8 tile rows) of A and of B (block blk = it*kWaves + wave);
  // LDS slot = lane, i.e. row r = 8*blk + lane/8 and stored chunk lane%8,
  // which holds logical chunk (lane%8) ^ ((r >> 1) & 7) =
  // (lane%8) ^ (lane/16) ^ 4*(blk&1), and blk&1 = wave&1 for every blk this
  // wave loads.
  const int lch = (lane & 7) ^ (lane >> 4) ^ (4 * (wave & 1));   // logical chunk this lane fetches
  const uint32_t va_off = (uint32_t)(lane >> 3) * lda + lch * 16;
  const uint32_t vb_off = (uint32_t)(lane >> 3) * ldb + lch * 16;
  // per-lane scale offsets: A row a_row0 + 128*wm + 32*mi + l32 is lane row
  // la = (a_row0 & 31) + l32 of 32-row group 4*wm + mi past the base
  const uint32_t la = (uint32_t)(a_row0 & 31) + l32;
  const uint32_t vsa_off = (la >> 5) * (uint32_t)sa.grp + (la & 31) * (uint32_t)sa.row;
  const uint32_t vsb_off = (uint32_t)l32 * (uint32_t)sb.row;
  // first 128-column step of this tile's k range in the scale layout
  const int q_base = MODE == MX_GROUP_K ? (args.k_tiled ? gt.q0[slot] : (int)(kbeg >> 7)) : 0;

  // valid A rows of this wave's 128 (wave-uniform; <= 0: none)
  const int wave_rows = __builtin_amdgcn_readfirstlane(a_rows_valid - (BM / 2) * wm);
  v16f acc[NS][4];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[s][mi][v] = 0.0f;

  // scales: raw words (dword path) or bytes of the next and current k-step
  uint32_t sb_n[NS][2], sa_n[4][2];
  uint32_t sb_c[NS][2], sa_c[4][2];

  // Scale loads of one k-step, in slices (slice p: sub-tile p of B for
  // p < NS, m sub-tile p-NS of A after), spread over the MFMA steps.
  auto load_scale_part = [&](int k0, int p) __attribute__((always_inline)) {
    const int blk0 = (int)((kbeg + k0) / 32);
    const __amdgpu_buffer_rsrc_t& rs = p < NS ? rsb : rsa;
    const uint32_t voff = p < NS ? vsb_off : vsa_off;
    const uint32_t so = p < NS ? (b_row_base(nsub(p)) >> 5) * (uint32_t)sb.grp
                               : (uint32_t)(4 * wm + (p - NS)) * (uint32_t)sa.grp;
    uint32_t* dst = p < NS ? sb_n[p] : sa_n[p - NS];
    if constexpr (SC != kScByte) {
      // the scale word of this k-step: blocks 4q .. 4q+3 of the row
      const uint32_t qo = (uint32_t)(q_base + (k0 >> 7)) * (uint32_t)(p < NS ? sb.step : sa.step);
      dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, so + qo, 0);
      dst[1] = 0;
    } else {
      // per-lane block index: blk0 + h (+2), clamped to the group's last block
      const uint32_t b0 = (uint32_t)min(blk0 + h, blk_last), b1 = (uint32_t)min(blk0 + 2 + h, blk_last);
      dst[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff + b0, so, 0);
      dst[1] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff + b1, so, 0);
    }
  };
  // Slice p (0..7) of the loads of k-step kt: block p of this wave's 1 KB
  // blocks (8 tile rows) of A and of B into the LDS stage (p < kDmaPerWave),
  // and the scales: slice p into registers (p < NS + 4), or for the k-tiled
  // layout one DMA per wave 0-2 at p = 0 into the LDS scale stage.
  auto load_part = [&](int kt, uint8_t* dA, uint8_t* dB, int p) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    if (p < kDmaPerWave) {
      const int blk = p * kWaves + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dA + blk * 1024), 16, va_off,
                                               (uint32_t)(8 * blk) * lda + k0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(dB + blk * 1024), 16, vb_off,
                                               b_row_base(8 * blk) * ldb + k0, 0, 0);
    }
    if constexpr (SC == kScLds) {
      // one k-step's words of 32 rows are 128 contiguous bytes: waves 0 and 1
      // fetch A row groups 0-7 and 8-15, wave 2 B row groups 0-7
      if (p == 0 && wave < 3) {
        const int st = (kt - kt_lo) & 1;
        const uint32_t c16 = (uint32_t)(lane & 7) * 16, g = (uint32_t)(lane >> 3);
        const uint32_t so = (uint32_t)(q_base + kt) * 128;
        if (wave < 2)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(sSc + st * kScStage + 256 * wave), 16,
                                                   (8 * wave + g) * (uint32_t)sa.grp + c16, so, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void*)(sSc + st * kScStage + 512), 16,
                                                   (b_row_base(32 * g) >> 5) * (uint32_t)sb.grp + c16, so, 0, 0);
      }
    } else {
      if (p < NS + 4) load_scale_part(k0, p);
    }
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
  // Hand the loaded scales of k-step kt to the MFMAs. Group-K scale words of a
  // group's last, partial k-step carry bytes of blocks past the group, which
  // are cleared (their codes are zero, but a NaN code would still poison the
  // products).
  auto take_scales = [&](int kt) __attribute__((always_inline)) {
    if constexpr (SC == kScLds) {
      // words of this lane's rows, from the stage of k-step kt (after the
      // barrier that follows its DMA)
      const uint32_t* ss = sSc + ((kt - kt_lo) & 1) * kScStage;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) { sa_n[mi][0] = ss[(a_row0 & 31) + 128 * wm + 32 * mi + l32]; sa_n[mi][1] = 0; }
#pragma unroll
      for (int s = 0; s < NS; ++s) { sb_n[s][0] = ss[512 + nsub(s) + l32]; sb_n[s][1] = 0; }
    }
    uint32_t m = 0xFFFFFFFFu;
    if constexpr (MODE == MX_GROUP_K && SC != kScByte) {
      const int rem = klen - kt * BK;
      m = rem >= BK ? 0xFFFFFFFFu : (rem <= 0 ? 0u : (1u << (8 * (rem >> 5))) - 1u);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) { sb_c[s][0] = sb_n[s][0] & m; sb_c[s][1] = sb_n[s][1]; }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) { sa_c[mi][0] = sa_n[mi][0] & m; sa_c[mi][1] = sa_n[mi][1]; }
  };
  // byte-0-aligned scale register of k-step ks: block h (ks 0) or 2+h (ks 1)
  auto scale_of = [&](uint32_t c0, uint32_t c1, int ks) __attribute__((always_inline)) -> int {
    if constexpr (SC != kScByte) return (int)(c0 >> (8 * h + 16 * ks));
    else return (int)(ks == 0 ? c0 : c1);
  };
  // MFMAs of one 128-wide k tile (2 MFMA k-steps x 4 m sub-tiles x NS n
  // sub-tiles) in 8 steps of NS MFMAs. Fragment reads run ahead of the MFMAs
  // that use them: A fragments two steps ahead (three registers sets), the B
  // fragments of k-step 1 one per step during k-step 0. Each step also issues
  // slices of the next k-step's loads (when: see the step body).
  auto compute = [&](const uint8_t* sA, const uint8_t* sB, int kt_next, uint8_t* nA, uint8_t* nB)
      __attribute__((always_inline)) {
    v8i fb_c[NS], fb_n[NS], fa[3];
    static_for<0, NS>([&](auto s_c) __attribute__((always_inline)) {
      constexpr int s = decltype(s_c)::value;
      fb_c[s] = read_frag(sB, nsub(s) + l32, 0);
    });
    fa[0] = read_frag(sA, 128 * wm + l32, 0);
    fa[1] = read_frag(sA, 128 * wm + 32 + l32, 0);
    static_for<0, 8>([&](auto step_c) __attribute__((always_inline)) {
      constexpr int step = decltype(step_c)::value;
      constexpr int ks = step / 4, mi = step % 4;
      // slice p of the next k-step's loads: at step p (group-K), or two
      // steps earlier (group-M: slices 0-2 at step 0, slice p at step p-2),
      // which gives the last slices more time to land before the hand-off
      // (measured: group-M GEMMs 1.5-3.6% faster, wgrad 1.5% slower)
      if constexpr (MODE == MX_GROUP_M) {
        if constexpr (step == 0) { load_part(kt_next, nA, nB, 0); load_part(kt_next, nA, nB, 1); }
        if constexpr (step + 2 < 8) load_part(kt_next, nA, nB, step + 2);
      } else {
        load_part(kt_next, nA, nB, step);
      }
      if constexpr (step + 2 < 8)
        fa[(step + 2) % 3] = read_frag(sA, 128 * wm + 32 * ((step + 2) % 4) + l32, (step + 2) / 4);
      if constexpr (step < NS) fb_n[step] = read_frag(sB, nsub(step) + l32, 1);
      // a 32-row block wholly past the tile's valid A rows (the last m-tile
      // of a group) keeps zero accumulators, which every epilogue masks or
      // drops anyway: its MFMAs are skipped (wave-uniform branch)
      if (32 * mi < wave_rows) {
        static_for<0, NS>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          acc[s][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              ks == 0 ? fb_c[s] : fb_n[s], fa[step % 3], acc[s][mi], 0, 0, 0,
              scale_of(sb_c[s][0], sb_c[s][1], ks), 0, scale_of(sa_c[mi][0], sa_c[mi][1], ks));
        });
      }
      // fence: each step's slice of loads stays with its 4 MFMAs
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Zero the chunks of a staged k-step that lie past klen (the k tail of a
  // group-K tile): each lane clears the LDS slots it loaded.
  auto zero_tail = [&](int kt, uint8_t* dA, uint8_t* dB) __attribute__((always_inline)) {
    const bool ok = kt * BK + lch * 16 < klen;
    if (!ok) {
#pragma unroll
      for (int it = 0; it < kDmaPerWave; ++it) {
        const int blk = it * kWaves + wave;
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
  // L2 prefetch: once a k-step's loads are issued, each wave touches one
  // 128-byte line per row of a share of the operand rows of k-step
  // kt + kPrefetchAhead, so that step's LDS loads hit L2 instead of waiting
  // for memory. The 32 tiles one XCD runs at a time (Bm m-tiles x 32/Bm
  // n-tiles of the band raster, Bm = band_m(MODE)) share A and B blocks, so a
  // tile touches only its share: A rows [8Bm*(nt%(32/Bm)), +8Bm) (waves 0-1,
  // half each) and B rows [(256/Bm)*(mt%Bm), +256/Bm) (waves 2-3, half
  // each). The loaded words land in a sink register one k-step later, when
  // the in-order completion of the next loads has made them ready, so the
  // prefetch never adds a wait.
  uint32_t pf_sink = 0, pf_last = 0;
  constexpr int Bm = band_m(MODE), SA = 8 * Bm, SB = 256 / Bm;
  const uint32_t pf_row = wave < 2 ? (uint32_t)(SA * (tc.nt % (32 / Bm)) + (SA / 2) * wave + (lane % (SA / 2)))
                                   : (uint32_t)(SB * (tc.mt % Bm) + (SB / 2) * (wave - 2) + (lane % (SB / 2)));
  const uint32_t pf_voff = wave < 2 ? pf_row * lda : b_row_base(pf_row & ~7u) * ldb + (pf_row & 7u) * ldb;
  auto prefetch = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    const uint32_t k0 = (uint32_t)kt * BK;
    return wave < 2 ? __builtin_amdgcn_raw_buffer_load_b32(ra, pf_voff, k0, 0)
                    : __builtin_amdgcn_raw_buffer_load_b32(rb, pf_voff, k0, 0);
  };
  auto kstep = [&](int kt, const uint8_t* cA, const uint8_t* cB, uint8_t* nA, uint8_t* nB)
      __attribute__((always_inline)) {
    compute(cA, cB, kt + 1, nA, nB);
    const uint32_t pf_new = prefetch(kt + kPrefetchAhead);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt1);     // all but the prefetch just issued
    if constexpr (SC == kScLds) {
      __syncthreads();
      take_scales(kt + 1);
    } else {
      take_scales(kt + 1);
      __syncthreads();
    }
    pf_sink ^= pf_last;
    pf_last = pf_new;
    if ((klen & (BK - 1)) != 0 && kt + 2 == kt_hi) {
      zero_tail(kt + 1, nA, nB);
      __syncthreads();
    }
  };

  if (kt_hi > kt_lo) {
    load_full(kt_lo, sA0, sB0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (SC == kScLds) {
      __syncthreads();
      take_scales(kt_lo);
    } else {
      take_scales(kt_lo);
      __syncthreads();
    }
    if ((klen & (BK - 1)) != 0 && kt_lo + 1 == kt_hi) {
      zero_tail(kt_lo, sA0, sB0);
      __syncthreads();
    }
  }
  // k-step kt_lo + j lives in stage j & 1
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    kstep(kt, sA0, sB0, sA1, sB1);
    if (kt + 1 < kt_hi) kstep(kt + 1, sA1, sB1, sA0, sB0);
  }

  asm volatile("" :: "v"(pf_sink ^ pf_last));

  // ---------------------------------------------------------------- epilogues
  // Lane mapping of the accumulators: for n sub-tile s and m sub-tile mi the
  // lane holds m_local = 128*wm + 32*mi + l32 and
  // n_local = nsub(s) + 8*(v/4) + 4*h + v%4 for v = 0..15.
  // Outputs go through buffer resources based at the wave's first row: the
  // offsets are 32-bit and rows past the valid ones fall outside the resource,
  // where stores are dropped and loads return 0. The per-lane indices are
  // re-derived from an opaque copy of the lane id so that no epilogue address
  // is computed before (and kept live across) the main loop.
  int lane_e = lane;
  asm volatile("" : "+v"(lane_e));
  {
  const int h = lane_e >> 5;        // shadows of the loop's lane-derived values
  const int l32 = lane_e & 31;
  const int tid = wave * 64 + lane_e;
  const int wrows = max(0, min(BM / 2, a_rows_valid - (BM / 2) * wm));   // valid rows of this wave
  const int64_t m0 = a_row0 + (BM / 2) * wm;                             // global row of its first row
  // wave-private 128 KB / kWaves of LDS: the k-loop's stages (4 x 32 KB) are
  // free after its last barrier
  constexpr int kSlice = 4 * BM * BK / kWaves;
  uint8_t* const slice = [&]() -> uint8_t* {
    const int a = wave * kSlice / (BM * BK), o = wave * kSlice % (BM * BK);
    return (a == 0 ? sA0 : a == 1 ? sA1 : a == 2 ? sB0 : sB1) + o;
  }();

  // 32 E4M3 codes of one row block, 4 dwords per lane (columns 8*vg + 4*h ..
  // +3): regroup over the half-waves so that lane half h holds columns
  // 16h .. 16h+15, then store them as one 16-byte run.
  auto store_row_codes = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off, const uint32_t (&q)[4])
      __attribute__((always_inline)) {
    const uint32_t r0 = xhalf(q[2], q[0], h), r1 = xhalf(q[3], q[1], h);
    u32x4 v;
    if (h) { v.x = r0; v.y = q[2]; v.z = r1; v.w = q[3]; }
    else   { v.x = q[0]; v.y = r0; v.z = q[1]; v.w = r1; }
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off + 16 * h, 0, 0);
  };
  // 32 bf16 values of one row (16 per lane, as above): lanes of the lower half
  // end with columns 0-7 and 16-23, the upper half with 8-15 and 24-31, so
  // each of the two stores writes 32 contiguous bytes per row.
  auto store_row_bf16 = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off, const float (&x)[16])
      __attribute__((always_inline)) {
    uint32_t p[4][2];
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      p[vg][0] = pack_bf16x2(x[4 * vg], x[4 * vg + 1]);
      p[vg][1] = pack_bf16x2(x[4 * vg + 2], x[4 * vg + 3]);
    }
    const uint32_t e0 = xhalf(p[1][0], p[0][0], h), e1 = xhalf(p[1][1], p[0][1], h);
    const uint32_t f0 = xhalf(p[3][0], p[2][0], h), f1 = xhalf(p[3][1], p[2][1], h);
    u32x4 a, b;
    if (h) { a.x = e0; a.y = e1; a.z = p[1][0]; a.w = p[1][1]; b.x = f0; b.y = f1; b.z = p[3][0]; b.w = p[3][1]; }
    else   { a.x = p[0][0]; a.y = p[0][1]; a.z = e0; a.w = e1; b.x = p[2][0]; b.y = p[2][1]; b.z = f0; b.w = f1; }
    __builtin_amdgcn_raw_buffer_store_b128(a, r, off + 16 * h, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, off + 32 + 16 * h, 0, 0);
  };
  // Both MXFP8 layouts of one 32 x 32 block of an fp32 intermediate d (this
  // lane: row l32 of the block, 16 columns). Rowwise: one scale per row over
  // the 32 columns (lanes l, l^32), codes stored directly. Columnwise: the
  // block is written transposed into the wave's fp32 area tr ([column][row],
  // kTrStride floats per column) and read back so that lane L holds rows
  // 16*(L/32) .. +15 of column L%32: the column amax is a local max plus one
  // exchange with lane L^32, and the 16 codes are 16 consecutive bytes of the
  // column's run in the columnwise layout, stored at
  // c_off + (L%32) * ldq + 16*(L/32) of rc when col_store.
  // The scale codes come back to the caller, which gathers the bytes that
  // share a k-tiled word and stores whole words: row_sc is the rowwise code
  // of this lane's row, col_sc the columnwise code of block column l32 (each
  // column once in the lanes with h == 0).
  auto quantize_block = [&](const float (&d)[16], const __amdgpu_buffer_rsrc_t& rq, uint32_t q_off,
                            bool row_store, float* tr, const __amdgpu_buffer_rsrc_t& rc, uint32_t c_off,
                            uint32_t ldq, bool col_store, uint32_t& row_sc, uint32_t& col_sc)
      __attribute__((always_inline)) {
    {
      uint32_t am = 0;
#pragma unroll
      for (int v = 0; v < 16; ++v) am = umax(am, abs_bits(d[v]));
      am = max_halves(am);
      const uint32_t sc = scale_code_from_amax_bits(am);
      const float inv = inv_scale_from_code(sc);
      uint32_t q[4];
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) q[vg] = e4m3x4(d[4 * vg] * inv, d[4 * vg + 1] * inv, d[4 * vg + 2] * inv, d[4 * vg + 3] * inv);
      if (row_store) store_row_codes(rq, q_off, q);
      row_sc = sc;
    }
    {
#pragma unroll
      for (int vg = 0; vg < 4; ++vg)
#pragma unroll
        for (int i = 0; i < 4; ++i) tr[(8 * vg + 4 * h + i) * kTrStride + l32] = d[4 * vg + i];
      float cv[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 t = *reinterpret_cast<const float4*>(tr + l32 * kTrStride + 16 * h + 4 * j);
        cv[4 * j] = t.x; cv[4 * j + 1] = t.y; cv[4 * j + 2] = t.z; cv[4 * j + 3] = t.w;
      }
      uint32_t am = 0;
#pragma unroll
      for (int v = 0; v < 16; ++v) am = umax(am, abs_bits(cv[v]));
      am = max_halves(am);
      const uint32_t sc = scale_code_from_amax_bits(am);
      const float inv = inv_scale_from_code(sc);
      u32x4 q;
      q.x = e4m3x4(cv[0] * inv, cv[1] * inv, cv[2] * inv, cv[3] * inv);
      q.y = e4m3x4(cv[4] * inv, cv[5] * inv, cv[6] * inv, cv[7] * inv);
      q.z = e4m3x4(cv[8] * inv, cv[9] * inv, cv[10] * inv, cv[11] * inv);
      q.w = e4m3x4(cv[12] * inv, cv[13] * inv, cv[14] * inv, cv[15] * inv);
      if (col_store) __builtin_amdgcn_raw_buffer_store_b128(q, rc, c_off + (uint32_t)l32 * ldq + 16 * h, 0, 0);
      col_sc = sc;
    }
  };
  if constexpr (EPI == EPI_F32 || EPI == EPI_BF16) {
    if (MODE == MX_GROUP_K && klen == 0 && args.accumulate) return;
    // fp32 out: the accumulators leave through the wave's LDS slice so that
    // every store covers whole 128-byte rows. 32 x 32 block (mi, s) is staged
    // as [row][16-byte chunk] (chunk c of row r at slot c ^ (r & 7), which
    // keeps both passes free of bank conflicts) and read back so that lane L
    // holds row 8i + L/8, chunk L%8 for i = 0..3; rd is based at the wave's
    // first row and column, ld is its row stride in floats, blocks from
    // column cols_valid on are skipped. Old values of an accumulating store
    // are read in the same layout. Accumulate and overwrite are separate code
    // paths so the accumulator registers never merge with the loaded values.
    const int rr = lane_e >> 3, cc = lane_e & 7;
    auto store_f32 = [&](const __amdgpu_buffer_rsrc_t& rd, uint32_t ld, int64_t cols_valid, auto acc_c,
                         auto policy_c) __attribute__((always_inline)) {
      constexpr bool ACC = decltype(acc_c)::value;
      constexpr int POL = decltype(policy_c)::value;
      auto coff = [&](int mi, int s, int i) __attribute__((always_inline)) -> uint32_t {
        return ((uint32_t)(32 * mi + 8 * i + rr) * ld + 32 * s + 4 * cc) * 4;
      };
      // Old values of an accumulating store: two 32-row blocks in flight (the
      // loads of block mi + 2 go out as soon as block mi has been added), so
      // the read latency is exposed once per tile rather than once per block.
      u32x4 old_e[NS][4], old_o[NS][4];
      auto load_old = [&](int mi, u32x4 (&o)[NS][4]) __attribute__((always_inline)) {
        static_for<0, NS * 4>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int s = decltype(j_c)::value / 4, i = decltype(j_c)::value % 4;
          o[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rd, coff(mi, s, i), 0, POL);
        });
      };
      if constexpr (ACC) {
        load_old(0, old_e);
        load_old(1, old_o);
      }
      static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
        constexpr int mi = decltype(mi_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        u32x4 (&old)[NS][4] = (mi & 1) ? old_o : old_e;
        uint8_t* const st = slice + (mi & 1) * (NS * 4096);
        static_for<0, NS * 4>([&](auto j_c) __attribute__((always_inline)) {
          constexpr int s = decltype(j_c)::value / 4, vg = decltype(j_c)::value % 4;
          u32x4 v;
          v.x = __float_as_uint(acc[s][mi][4 * vg + 0]); v.y = __float_as_uint(acc[s][mi][4 * vg + 1]);
          v.z = __float_as_uint(acc[s][mi][4 * vg + 2]); v.w = __float_as_uint(acc[s][mi][4 * vg + 3]);
          const int c = 2 * vg + h;
          *reinterpret_cast<u32x4*>(st + s * 4096 + l32 * 128 + ((c ^ (l32 & 7)) << 4)) = v;
        });
        static_for<0, NS>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          if (32 * s < cols_valid) {
            static_for<0, 4>([&](auto i_c) __attribute__((always_inline)) {
              constexpr int i = decltype(i_c)::value;
              u32x4 v = *reinterpret_cast<const u32x4*>(st + s * 4096 + (8 * i + rr) * 128 + ((cc ^ rr) << 4));
              if constexpr (ACC) {
                v.x = __float_as_uint(__uint_as_float(v.x) + __uint_as_float(old[s][i].x));
                v.y = __float_as_uint(__uint_as_float(v.y) + __uint_as_float(old[s][i].y));
                v.z = __float_as_uint(__uint_as_float(v.z) + __uint_as_float(old[s][i].z));
                v.w = __float_as_uint(__uint_as_float(v.w) + __uint_as_float(old[s][i].w));
              }
              __builtin_amdgcn_raw_buffer_store_b128(v, rd, coff(mi, s, i), 0, POL);
            });
          }
        });
        if constexpr (ACC && mi + 2 < 4) {
          __builtin_amdgcn_sched_barrier(0);
          load_old(mi + 2, old);
        }
      });
    };
    using plain = std::integral_constant<int, 0>;
    using once = std::integral_constant<int, kNonTemporal>;
    if (MODE == MX_GROUP_M && split_unit >= 0) {
      // split-K part: the whole 256 x 256 fp32 partial, row-major, into its
      // workspace slot (the reduce kernel adds the parts and writes C)
      const __amdgpu_buffer_rsrc_t rw =
          make_rsrc(args.split_ws + (int64_t)split_unit * BM * BN + (BM / 2) * wm * BN + kWaveN * wn,
                    (int64_t)(BM / 2) * BN * 4);
      store_f32(rw, BN, BN, std::false_type{}, plain{});
      return;
    }
    constexpr int esz = EPI == EPI_F32 ? 4 : 2;
    const uint32_t ldc = (uint32_t)args.ldc;
    const int64_t col0 = (int64_t)tc.nt * BN + kWaveN * wn;
    const char* cb = reinterpret_cast<const char*>(args.c);
    if constexpr (MODE == MX_GROUP_K) cb += (int64_t)g * args.c_group_stride * esz;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cb + (m0 * args.ldc + col0) * esz, (int64_t)wrows * args.ldc * esz);
    if constexpr (EPI == EPI_F32) {
      // C is touched once: non-temporal
      if (args.accumulate) store_f32(rc, ldc, args.N - col0, std::true_type{}, once{});
      else store_f32(rc, ldc, args.N - col0, std::false_type{}, once{});
    } else {
      static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
        constexpr int mi = decltype(mi_c)::value;
        static_for<0, NS>([&](auto s_c) __attribute__((always_inline)) {
          constexpr int s = decltype(s_c)::value;
          __builtin_amdgcn_sched_barrier(0);
          if (col0 + 32 * s < args.N) {
            float x[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) x[v] = acc[s][mi][v];
            store_row_bf16(rc, ((uint32_t)(32 * mi + l32) * ldc + 32 * s) * 2, x);
          }
        });
      });
    }
  } else if constexpr (EPI == EPI_SWIGLU_FWD) {
    // gate (sub-tile s) and up (s + NS/2), s < NS/2, of ffn columns
    // j = jw0 + 32*s + 8*(v/4) + 4*h + v%4; a = w * silu(gate) * up.
    const uint32_t F = (uint32_t)args.F;
    const int jw0 = tc.nt * (BN / 2) + (NS / 2) * 32 * wn;
    const int wrow0 = tc.mt * BM + (BM / 2) * wm;       // first row of the wave inside its group
    const int len = gt.len[slot];
    const uint32_t ldq = (uint32_t)args.ld_col;
    const int64_t crow0 = gt.pc0[slot] + wrow0;   // columnwise position of the wave's first row
    const __amdgpu_buffer_rsrc_t rprob = make_rsrc(args.probs ? args.probs + m0 : nullptr, args.probs ? (int64_t)wrows * 4 : 0);
    const __amdgpu_buffer_rsrc_t rh1 = make_rsrc(args.h1 ? args.h1 + m0 * 2 * F : nullptr, args.h1 ? (int64_t)wrows * 4 * F : 0);
    const __amdgpu_buffer_rsrc_t rqr = make_rsrc(args.q_row + m0 * F, (int64_t)wrows * F);
    const __amdgpu_buffer_rsrc_t rsr = make_rsrc(args.s_row, (int64_t)((args.R + 31) >> 5) * args.nq_row * 128);
    const bool col_out = args.q_col != nullptr;
    const __amdgpu_buffer_rsrc_t rqc = make_rsrc(col_out ? args.q_col + (int64_t)jw0 * ldq + crow0 : nullptr,
                                                 col_out ? (int64_t)(NS / 2) * 32 * ldq : 0);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(col_out ? args.s_col : nullptr,
                                                 col_out ? (int64_t)(F >> 5) * args.nq_col * 128 : 0);
    const uint32_t q0 = (uint32_t)gt.q0[slot];
    // routing weights of the lane's 4 rows: the loads go out together and
    // unconditionally (without probs the resource is empty and they read 0),
    // the choice comes after, so no load waits at a branch join
    float w[4], wl[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) wl[mi] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rprob, 4 * (32 * mi + l32), 0, 0));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) w[mi] = args.probs ? wl[mi] : (32 * mi + l32 < wrows ? 1.0f : 0.0f);
    // Scale words: the wave's NS/2 column blocks are bytes 2*wn .. of one
    // rowwise word per row, and its 4 row blocks the 4 bytes of one
    // columnwise word per column (bytes of blocks past the group are 0).
    const uint32_t b0 = (uint32_t)jw0 >> 5;
    const bool wave_jok = jw0 < (int)F;                  // F % 128 == 0: all NS/2 blocks valid or none
    uint32_t csw[NS / 2];
#pragma unroll
    for (int s2 = 0; s2 < NS / 2; ++s2) csw[s2] = 0;
    static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
      constexpr int mi = decltype(mi_c)::value;
      const uint32_t r = 32 * mi + l32;
      const bool blk_ok = col_out && wrow0 + 32 * mi < len;
      uint32_t rsw = 0;
      static_for<0, NS / 2>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        const bool jok = jw0 + 32 * s < (int)F;          // F % 32 == 0: whole block valid or not
        // rows past the group's end are forced to 0 (they share columnwise
        // blocks with valid rows up to the 32-row padding)
        const bool rv = r < (uint32_t)wrows;
        float gv[16], uv[16], a[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          gv[v] = vgpr_hop(acc[s][mi][v]);
          uv[v] = vgpr_hop(acc[s + NS / 2][mi][v]);
          const float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[v]));
          a[v] = rv ? w[mi] * (gv[v] * sig) * uv[v] : 0.0f;
        }
        if (args.h1 != nullptr && jok) {
          store_row_bf16(rh1, (r * 2 * F + jw0 + 32 * s) * 2, gv);
          store_row_bf16(rh1, (r * 2 * F + F + jw0 + 32 * s) * 2, uv);
        }
        uint32_t rsc_v, csc_v;
        quantize_block(a, rqr, r * F + jw0 + 32 * s, jok, reinterpret_cast<float*>(slice), rqc,
                       (uint32_t)(32 * s) * ldq + 32 * mi, ldq, jok && blk_ok, rsc_v, csc_v);
        rsw |= rsc_v << (8 * s);
        csw[s] |= (blk_ok ? csc_v : 0u) << (8 * mi);
      });
      {
        const uint32_t m = (uint32_t)m0 + r;             // global row
        if (wave_jok && r < (uint32_t)wrows && h == 0)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)rsw, rsr,
                                                ((m >> 5) * args.nq_row + (b0 >> 2)) * 128 + (m & 31) * 4 + (b0 & 3), 0, 0);
      }
    });
    // columnwise scale words: only where the wave has rows of the group (the
    // word past the group's last k-step belongs to the next group)
    if (col_out && wave_jok && wrow0 < len && h == 0) {
#pragma unroll
      for (int s2 = 0; s2 < NS / 2; ++s2)
        __builtin_amdgcn_raw_buffer_store_b32(csw[s2], rsc,
                                              ((b0 + s2) * args.nq_col + q0 + ((uint32_t)wrow0 >> 7)) * 128 + l32 * 4,
                                              0, 0);
    }
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // acc = dA for ffn columns j = jw0 + 32*s + 8*(v/4) + 4*h + v%4 (s = 0..3)
    __shared__ float red[kWavesN * BM];
    const uint32_t F = (uint32_t)args.F;
    const int jw0 = tc.nt * BN + kWaveN * wn;
    const int wrow0 = tc.mt * BM + (BM / 2) * wm;
    const int len = gt.len[slot];
    const uint32_t ldq = (uint32_t)args.ld_col;
    const int64_t crow0 = gt.pc0[slot] + wrow0;
    const __amdgpu_buffer_rsrc_t rprob = make_rsrc(args.probs ? args.probs + m0 : nullptr, args.probs ? (int64_t)wrows * 4 : 0);
    const __amdgpu_buffer_rsrc_t rh1 = make_rsrc(args.h1 + m0 * 2 * F, (int64_t)wrows * 4 * F);
    const __amdgpu_buffer_rsrc_t rqr = make_rsrc(args.q_row + m0 * 2 * F, (int64_t)wrows * 2 * F);
    const __amdgpu_buffer_rsrc_t rsr = make_rsrc(args.s_row, (int64_t)((args.R + 31) >> 5) * args.nq_row * 128);
    // columnwise dH1: gate half (columns j) and up half (columns F + j)
    const __amdgpu_buffer_rsrc_t rqc_g = make_rsrc(args.q_col + (int64_t)jw0 * ldq + crow0, (int64_t)kWaveN * ldq);
    const __amdgpu_buffer_rsrc_t rqc_u = make_rsrc(args.q_col + (int64_t)(F + jw0) * ldq + crow0, (int64_t)kWaveN * ldq);
    const __amdgpu_buffer_rsrc_t rsc = make_rsrc(args.s_col, (int64_t)(2 * F >> 5) * args.nq_col * 128);
    const uint32_t q0 = (uint32_t)gt.q0[slot];
    // routing weights of the lane's 4 rows: the loads go out together and
    // unconditionally (without probs the resource is empty and they read 0),
    // the choice comes after, so no load waits at a branch join
    float w[4], wl[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) wl[mi] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rprob, 4 * (32 * mi + l32), 0, 0));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) w[mi] = args.probs ? wl[mi] : (32 * mi + l32 < wrows ? 1.0f : 0.0f);
    float dpsum[4];
    // Scale words: the wave's NS column blocks of the gate (and of the up)
    // half are the 4 bytes of one rowwise word per row, and its 4 row blocks
    // the 4 bytes of one columnwise word per column (bytes of blocks past the
    // group are 0). The columnwise bytes collect in the slice past the
    // transpose area, word (half, s, column).
    const uint32_t bg0 = (uint32_t)jw0 >> 5, bu0 = (uint32_t)(F + jw0) >> 5;
    const bool wave_jok = jw0 < (int)F;                  // F % 128 == 0: all NS blocks valid or none
    static_assert(kTrBytes + 2 * NS * 32 * 4 <= kSlice, "column scale bytes must fit the wave's slice");
    uint8_t* const csl = slice + kTrBytes;
    // gate and up (bf16) of one 32-row block and 32 columns (16 per lane) are
    // a unit of 8 loads; a ring of NS units keeps the next NS units in flight
    // (unit (mi + 1, s) is requested once unit (mi, s) has been used), so the
    // H1 read latency is exposed once per tile rather than once per row block.
    u32x2 gl[NS][4], ul[NS][4];
    auto load_gu = [&](int mi, int s) __attribute__((always_inline)) {
      const uint32_t r = 32 * mi + l32;
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const uint32_t o = (r * 2 * F + jw0 + 32 * s + 8 * vg + 4 * h) * 2;
        gl[s][vg] = __builtin_amdgcn_raw_buffer_load_b64(rh1, o, 0, 0);
        ul[s][vg] = __builtin_amdgcn_raw_buffer_load_b64(rh1, o + 2 * F, 0, 0);
      }
    };
#pragma unroll
    for (int s = 0; s < NS; ++s) load_gu(0, s);
    static_for<0, 4>([&](auto mi_c) __attribute__((always_inline)) {
      constexpr int mi = decltype(mi_c)::value;
      const uint32_t r = 32 * mi + l32;
      const bool blk_ok = wrow0 + 32 * mi < len;
      uint32_t rsg = 0, rsu = 0;
      float dp = 0.0f;
      static_for<0, NS>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int s = decltype(s_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        const bool jok = jw0 + 32 * s < (int)F;
        const bool rv = r < (uint32_t)wrows;
        float dg[16], du[16];
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const float gv[4] = {bf16_lo(gl[s][vg].x), bf16_hi(gl[s][vg].x), bf16_lo(gl[s][vg].y), bf16_hi(gl[s][vg].y)};
          const float uv[4] = {bf16_lo(ul[s][vg].x), bf16_hi(ul[s][vg].x), bf16_lo(ul[s][vg].y), bf16_hi(ul[s][vg].y)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float da = vgpr_hop(acc[s][mi][4 * vg + i]);
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[i]));
            const float sl = gv[i] * sg;
            dg[4 * vg + i] = rv ? da * w[mi] * uv[i] * sg * (1.0f + gv[i] * (1.0f - sg)) : 0.0f;
            du[4 * vg + i] = rv ? da * w[mi] * sl : 0.0f;
            dp += jok ? da * sl * uv[i] : 0.0f;
          }
        }
        float* const tr = reinterpret_cast<float*>(slice);
        const uint32_t co = (uint32_t)(32 * s) * ldq + 32 * mi;
        uint32_t rg, cg, ru, cu;
        quantize_block(dg, rqr, r * 2 * F + jw0 + 32 * s, jok, tr, rqc_g, co, ldq, jok && blk_ok, rg, cg);
        quantize_block(du, rqr, r * 2 * F + F + jw0 + 32 * s, jok, tr, rqc_u, co, ldq, jok && blk_ok, ru, cu);
        rsg |= rg << (8 * s);
        rsu |= ru << (8 * s);
        if (h == 0) {
          csl[(s * 32 + l32) * 4 + mi] = (uint8_t)(blk_ok ? cg : 0u);
          csl[((NS + s) * 32 + l32) * 4 + mi] = (uint8_t)(blk_ok ? cu : 0u);
        }
        if constexpr (mi + 1 < 4) load_gu(mi + 1, s);
      });
      {
        const uint32_t m = (uint32_t)m0 + r;
        const uint32_t srow = (m >> 5) * args.nq_row * 128 + (m & 31) * 4;
        if (wave_jok && r < (uint32_t)wrows && h == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(rsg, rsr, srow + (bg0 >> 2) * 128, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(rsu, rsr, srow + (bu0 >> 2) * 128, 0, 0);
        }
      }
      dpsum[mi] = sum_halves(dp);
    });
    // columnwise scale words: only where the wave has rows of the group (the
    // word past the group's last k-step belongs to the next group)
    if (wave_jok && wrow0 < len && h == 0) {
      const uint32_t qo = q0 + ((uint32_t)wrow0 >> 7);
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        const uint32_t wg = *reinterpret_cast<const uint32_t*>(csl + (s2 * 32 + l32) * 4);
        const uint32_t wu = *reinterpret_cast<const uint32_t*>(csl + ((NS + s2) * 32 + l32) * 4);
        __builtin_amdgcn_raw_buffer_store_b32(wg, rsc, ((bg0 + s2) * args.nq_col + qo) * 128 + l32 * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(wu, rsc, ((bu0 + s2) * args.nq_col + qo) * 128 + l32 * 4, 0, 0);
      }
    }
    // dprobs partial over this tile's 256 columns: the n-waves meet in LDS
    if (args.dprobs_part != nullptr) {
      if (h == 0) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) red[wn * BM + (BM / 2) * wm + 32 * mi + l32] = dpsum[mi];
      }
      __syncthreads();
      if (tid < a_rows_valid) {
        float tot = red[tid];
#pragma unroll
        for (int w = 1; w < kWavesN; ++w) tot += red[w * BM + tid];
        args.dprobs_part[(int64_t)tc.nt * args.R + a_row0 + tid] = tot;
      }
    }
  }
  }  // epilogue scope
#endif  // __HIP_DEVICE_COMPILE__
}

// dprobs[r] = sum over p of part[p][r]. A workgroup takes 32 rows, its 256
// threads as 8 groups of 32 consecutive rows (coalesced 128-byte reads); group
// g sums parts g, g + 8, ... in order and the 8 group sums meet in LDS, added
// in group order, so the result is deterministic. (One thread per row left
// R / 256 workgroups, each thread with n_parts dependent loads: about 84 GB/s.)
constexpr int kDpRows = 32, kDpGroups = 8;
__global__ __launch_bounds__(256) void dprobs_reduce_kernel(const float* part, float* out, int32_t R, int32_t n_parts,
                                                            const int32_t* rows_dev) {
  __shared__ float red[kDpGroups][kDpRows];
  const int g = threadIdx.x / kDpRows, rl = threadIdx.x % kDpRows;
  const int r = blockIdx.x * kDpRows + rl;
  const int rows = rows_dev != nullptr ? min(R, *rows_dev) : R;   // rows past the routed ones get 0
  float s = 0.0f;
  if (r < rows) {
#pragma unroll 4
    for (int p = g; p < n_parts; p += kDpGroups) s += part[(int64_t)p * R + r];
  }
  red[g][rl] = s;
  __syncthreads();
  if (g == 0 && r < R) {
    float t = red[0][rl];
#pragma unroll
    for (int k = 1; k < kDpGroups; ++k) t += red[k][rl];
    out[r] = t;
  }
}

// Split-K tail: tile args.split_f + blockIdx.x is the sum of its
// args.split_s fp32 partials (added in part order); write it as C (bf16, or
// fp32 with optional accumulate) over the tile's valid rows and columns.
// Split-K reduce: one workgroup per kRedRows-row slab of a tail tile. A
// thread issues all of its loads (4 float4 positions x up to kMaxSplitParts
// parts) before adding, and adds the parts in part order (then the old value
// when accumulating), so the sums are those of a plain loop over the parts.
constexpr int kRedRows = 16;
template <int EPI>
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmArgs args) {
  constexpr int kSlabs = BM / kRedRows;
  static_assert(kRedRows * BN == 4 * 4 * 256, "a slab is 4 float4 per thread");
  const int tile = (int)blockIdx.x / kSlabs, slab = (int)blockIdx.x % kSlabs;
  const int id = args.split_f + tile;
  const TileCoord tc = locate_tile(args.groups, id, MX_GROUP_M, args.M, args.n_tiles_n);
  const int slot = tc.slot;
  const int64_t a_row0 = (int64_t)args.groups.a0[slot] + (int64_t)tc.mt * BM;
  const int rows_valid = min(BM, args.groups.len[slot] - tc.mt * BM);
  const int64_t col0 = (int64_t)tc.nt * BN;
  const int S = args.split_s;
  const float* ws = args.split_ws + (int64_t)tile * S * BM * BN + slab * kRedRows * BN;
  float4 v[kMaxSplitParts][4];
#pragma unroll
  for (int p = 0; p < kMaxSplitParts; ++p)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (p < S) v[p][k] = *reinterpret_cast<const float4*>(ws + (int64_t)p * BM * BN + (k * 256 + (int)threadIdx.x) * 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = (k * 256 + (int)threadIdx.x) * 4;
    const int r = slab * kRedRows + e / BN, c = e % BN;
    float4 sum = v[0][k];
#pragma unroll
    for (int p = 1; p < kMaxSplitParts; ++p)
      if (p < S) { sum.x += v[p][k].x; sum.y += v[p][k].y; sum.z += v[p][k].z; sum.w += v[p][k].w; }
    if (r >= rows_valid || col0 + c >= args.N) continue;
    const int64_t o = (a_row0 + r) * args.ldc + col0 + c;
    if constexpr (EPI == EPI_BF16) {
      uint2 w;
      w.x = pack_bf16x2(sum.x, sum.y);
      w.y = pack_bf16x2(sum.z, sum.w);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(args.c) + o) = w;
    } else {
      float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(args.c) + o);
      if (args.accumulate) {
        const float4 old = *d;
        sum.x += old.x; sum.y += old.y; sum.z += old.z; sum.w += old.w;
      }
      *d = sum;
    }
  }
}

template <int MODE, int EPI>
static hipError_t launch_mode_epi(bool svec, const GemmArgs& args, int total, hipStream_t stream) {
  if (args.groups_dev != nullptr) {
    // device-built group tables: k-tiled scales, no split-K tail
    if (!args.k_tiled || args.split_s > 1) return hipErrorInvalidValue;
    if constexpr ((MODE == MX_GROUP_M && EPI != EPI_F32) || (MODE == MX_GROUP_K && EPI == EPI_F32))
      hipLaunchKernelGGL((gemm_kernel<MODE, EPI, kScLds, true>), dim3(total), dim3(kThreads), 0, stream, args, total);
    else
      return hipErrorInvalidValue;
  } else if (args.k_tiled) {
    hipLaunchKernelGGL((gemm_kernel<MODE, EPI, kScLds, false>), dim3(total), dim3(kThreads), 0, stream, args, total);
  } else if constexpr (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD) {
    return hipErrorInvalidValue;       // the fused epilogues run on k-tiled scales only
  } else if (svec) {
    hipLaunchKernelGGL((gemm_kernel<MODE, EPI, kScDword, false>), dim3(total), dim3(kThreads), 0, stream, args, total);
  } else {
    hipLaunchKernelGGL((gemm_kernel<MODE, EPI, kScByte, false>), dim3(total), dim3(kThreads), 0, stream, args, total);
  }
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
      case EPI_F32: return launch_mode_epi<MX_GROUP_K, EPI_F32>(scale_dword, args, total_tiles, stream);
      case EPI_BF16: return launch_mode_epi<MX_GROUP_K, EPI_BF16>(scale_dword, args, total_tiles, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(int epi, const GemmArgs& args, int tail_tiles, hipStream_t stream) {
  if (tail_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)(tail_tiles * (BM / kRedRows)));
  if (epi == EPI_BF16)
    hipLaunchKernelGGL(split_reduce_kernel<EPI_BF16>, grid, dim3(256), 0, stream, args);
  else if (epi == EPI_F32)
    hipLaunchKernelGGL(split_reduce_kernel<EPI_F32>, grid, dim3(256), 0, stream, args);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dprobs_reduce(const float* part, float* dprobs, int32_t R, int32_t n_parts, const int32_t* rows_dev,
                                hipStream_t stream) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(dprobs_reduce_kernel, dim3((R + kDpRows - 1) / kDpRows), dim3(256), 0, stream, part, dprobs, R,
                     n_parts, rows_dev);
  return hipGetLastError();
}

}  // namespace mx
