// Host side of the C ABI declared in include/mxfp8.h: argument validation
// (before anything is enqueued), group/tile planning from the host
// split_sizes, buffer layout of the fused MLP, and kernel launches on the
// caller's stream. No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "mx_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local void* const* g_events = nullptr;   // optional stage-timing events
thread_local int32_t g_n_events = 0;

void stage_mark(int i, hipStream_t stream) {
  if (g_events != nullptr && i < g_n_events && g_events[i] != nullptr)
    (void)hipEventRecord(reinterpret_cast<hipEvent_t>(g_events[i]), stream);
}

mx_status fail(mx_status s, const char* fmt, ...);
mx_status hip_fail(hipError_t e, const char* what);

// Side stream of the calling thread on the current device, with the events
// that fork it from and join it back into the caller's stream. The fused MLP
// runs its HBM-bound stages there (the W2 cast, the wgrad GEMMs) beside the
// MFMA-bound ones; every side launch is ordered after the caller's earlier
// work and before its later work by these events, so to the caller all work
// is ordered on its own stream. Created on first use, default priority, kept
// for the life of the process; one set per thread so that calls from
// different threads never share an event.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
};
thread_local SideStream g_side[64];

mx_status side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MX_EUNSUPPORTED, "device index %d out of range", dev);
  SideStream& sd = g_side[dev];
  if (sd.s == nullptr) {
    e = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking);
    if (e != hipSuccess) { sd.s = nullptr; return hip_fail(e, "side stream"); }
    for (hipEvent_t& v : sd.ev) {
      e = hipEventCreateWithFlags(&v, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "side stream event");
    }
  }
  *out = &sd;
  return MX_OK;
}

// `to` waits for all work enqueued so far on `from` (event ev recorded on from).
mx_status wait_for(hipStream_t to, hipStream_t from, hipEvent_t ev) {
  hipError_t e = hipEventRecord(ev, from);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = hipStreamWaitEvent(to, ev, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  return MX_OK;
}

mx_status fail(mx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mx_status hip_fail(hipError_t e, const char* what) {
  return fail(MX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kI32Max = 0x7FFFFFFF;

int64_t pad32(int64_t m) { return (m + 31) / 32 * 32; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// k-tiled scales of a columnwise layout with row groups: first 128-column
// step of each group (q0[n] = total steps).
std::vector<int64_t> group_steps(const int64_t* sizes, int32_t n, int64_t rows) {
  std::vector<int64_t> q0(1, 0);
  const int ng = n > 0 ? n : 1;
  for (int g = 0; g < ng; ++g) q0.push_back(q0.back() + cdiv(pad32(n > 0 ? sizes[g] : rows), 128));
  return q0;
}

// ---------------------------------------------------------------- quantize
mx_status check_groups(const int64_t* sizes, int32_t n, int64_t rows, const char* who) {
  if (n < 0) return fail(MX_EINVAL, "%s: negative group count", who);
  if (n > mx::kMaxGroups) return fail(MX_EUNSUPPORTED, "%s: %d groups exceeds the maximum %d", who, n, mx::kMaxGroups);
  if (n > 0 && sizes == nullptr) return fail(MX_EINVAL, "%s: group sizes pointer is null", who);
  int64_t s = 0;
  for (int32_t g = 0; g < n; ++g) {
    if (sizes[g] < 0) return fail(MX_ESHAPE, "%s: group %d has negative size %lld", who, g, (long long)sizes[g]);
    s += sizes[g];
  }
  if (n > 0 && s != rows) return fail(MX_ESHAPE, "%s: group sizes sum to %lld, expected %lld", who, (long long)s, (long long)rows);
  return MX_OK;
}

// tiled: scales of both copies in the k-tiled layout (the fused MLP's
// internal buffers; needs cols % 128 == 0 for the rowwise copy).
// Device-built row groups for an activation cast of the fused MLP: the table,
// the worst-case layout of the columnwise copy and the worst-case row tiles.
struct DevQuant {
  const mx::QuantGroups* groups;
  int64_t ld_col;
  int32_t nq_col;
  int64_t row_tiles;
};

mx_status quantize_impl(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const int64_t* group_sizes,
                        int32_t num_groups, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                        hipStream_t stream, bool tiled = false, const int32_t* row_index = nullptr,
                        int64_t index_rows = 0, const DevQuant* dq = nullptr) {
  const char* who = "mx_quantize";
  if (x == nullptr) return fail(MX_EINVAL, "%s: x is null", who);
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return fail(MX_EINVAL, "%s: unsupported dtype %d", who, x_dtype);
  if ((q_row == nullptr) != (s_row == nullptr)) return fail(MX_EINVAL, "%s: rowwise codes and scales must both be given or both null", who);
  if ((q_col == nullptr) != (s_col == nullptr)) return fail(MX_EINVAL, "%s: columnwise codes and scales must both be given or both null", who);
  if (q_row == nullptr && q_col == nullptr) return fail(MX_EINVAL, "%s: no output requested", who);
  if (rows < 0 || cols <= 0) return fail(MX_ESHAPE, "%s: bad shape [%lld, %lld]", who, (long long)rows, (long long)cols);
  if (cols % 32) return fail(MX_ESHAPE, "%s: cols=%lld is not a multiple of 32", who, (long long)cols);
  if (rows > kI32Max || cols > kI32Max) return fail(MX_EUNSUPPORTED, "%s: dimension exceeds 2^31-1", who);
  if (num_groups == 0 && group_sizes != nullptr) return fail(MX_EINVAL, "%s: group sizes given with num_groups == 0", who);
  mx_status st = check_groups(group_sizes, num_groups, rows, who);
  if (st != MX_OK) return st;
  if (!aligned(x, 16) || (q_row && !aligned(q_row, 16)) || (q_col && !aligned(q_col, 16)))
    return fail(MX_EALIGN, "%s: x, q_row and q_col must be 16-byte aligned", who);

  mx::QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.q_row = q_row;
  a.s_row = s_row;
  a.q_col = q_col;
  a.s_col = s_col;
  a.cols = cols;
  const int n = num_groups > 0 ? num_groups : 1;
  a.groups.n = n;
  int64_t r0 = 0, p0 = 0, t0 = 0;
  for (int g = 0; g < n; ++g) {
    const int64_t m = num_groups > 0 ? group_sizes[g] : rows;
    a.groups.row0[g] = (int32_t)r0;
    a.groups.pcol0[g] = (int32_t)p0;
    a.groups.tile0[g] = (int32_t)t0;
    r0 += m;
    p0 += pad32(m);
    t0 += cdiv(m, mx::kQuantTileRows);
  }
  a.groups.row0[n] = (int32_t)r0;
  a.groups.pcol0[n] = (int32_t)p0;
  a.groups.tile0[n] = (int32_t)t0;
  if (tiled) {
    if (q_row != nullptr && cols % 128) return fail(MX_ESHAPE, "%s: k-tiled scales need cols %% 128 == 0", who);
    const std::vector<int64_t> q0 = group_steps(group_sizes, num_groups, rows);
    for (int g = 0; g <= n; ++g) a.groups.q0[g] = (int32_t)q0[g];
    a.tiled = 1;
    a.nq_row = (int32_t)(cols / 128);
    a.nq_col = (int32_t)q0[n];
    a.rows = (int32_t)rows;
  }
  a.row_index = row_index;
  a.index_rows = (int32_t)index_rows;
  if (p0 > kI32Max) return fail(MX_EUNSUPPORTED, "%s: padded rows exceed 2^31-1", who);
  a.ld_col = p0;
  a.n_col_tiles = (int32_t)cdiv(cols, mx::quant_tile_cols(x_dtype));
  if (dq != nullptr) {
    a.groups_dev = dq->groups;
    a.ld_col = dq->ld_col;
    a.nq_col = dq->nq_col;
    t0 = dq->row_tiles;
  }
  if (t0 * a.n_col_tiles > kI32Max) return fail(MX_EUNSUPPORTED, "%s: too many tiles", who);
  hipError_t e = mx::launch_quantize(a, x_dtype, (int)t0, stream);
  if (e != hipSuccess) return hip_fail(e, "mx_quantize launch");
  return MX_OK;
}

// ---------------------------------------------------------------- grouped GEMM
struct GemmPlan {
  mx::GemmArgs args;
  int total_tiles;
  bool scale_dword;
};

mx_status gemm_plan(int32_t mode, int32_t G, const int64_t* sizes, int64_t M, int64_t N, int64_t K,
                    const uint8_t* a, const uint8_t* as, int64_t lda, const uint8_t* b, const uint8_t* bs,
                    int64_t ldb, int64_t b_group_stride, void* c, int32_t c_dtype, int64_t ldc,
                    int64_t c_group_stride, int32_t accumulate, int epi, int64_t n_rows_b, GemmPlan* plan) {
  const char* who = "mx_grouped_gemm";
  if (mode != MX_GROUP_M && mode != MX_GROUP_K) return fail(MX_EINVAL, "%s: bad mode %d", who, mode);
  if (G < 1) return fail(MX_EINVAL, "%s: need at least one group", who);
  if (G > mx::kMaxGroups) return fail(MX_EUNSUPPORTED, "%s: %d groups exceeds the maximum %d", who, G, mx::kMaxGroups);
  if (!sizes) return fail(MX_EINVAL, "%s: sizes is null", who);
  if (!a || !as || !b || !bs || !c) return fail(MX_EINVAL, "%s: null operand pointer", who);
  if (c_dtype != MX_F32 && c_dtype != MX_BF16) return fail(MX_EINVAL, "%s: bad output dtype %d", who, c_dtype);
  if (accumulate && c_dtype != MX_F32) return fail(MX_EUNSUPPORTED, "%s: accumulate needs an fp32 output", who);
  if (M < 0 || N <= 0 || K < 0) return fail(MX_ESHAPE, "%s: bad sizes M=%lld N=%lld K=%lld", who, (long long)M, (long long)N, (long long)K);
  if (M > kI32Max || N > kI32Max || K > kI32Max) return fail(MX_EUNSUPPORTED, "%s: dimension exceeds 2^31-1", who);
  if (K % 32 || N % 32) return fail(MX_ESHAPE, "%s: K and N must be multiples of 32 (K=%lld N=%lld)", who, (long long)K, (long long)N);
  if (lda % 32 || ldb % 32 || lda < K || ldb < K) return fail(MX_ESHAPE, "%s: lda/ldb must be multiples of 32 and >= K", who);
  if (ldc < N || ldc % 4) return fail(MX_ESHAPE, "%s: ldc must be >= N and a multiple of 4", who);
  if (b_group_stride < 0 || b_group_stride % 32) return fail(MX_ESHAPE, "%s: b_group_stride must be a non-negative multiple of 32", who);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return fail(MX_EALIGN, "%s: a, b and c must be 16-byte aligned", who);
  // the kernels address one B group and one 256-row A tile with 32-bit offsets
  if (N * ldb >= (int64_t(1) << 32) || int64_t(mx::kTileM) * lda >= (int64_t(1) << 32))
    return fail(MX_EUNSUPPORTED, "%s: one B group or A tile exceeds 4 GiB", who);
  int64_t sum = 0, sumP = 0;
  for (int g = 0; g < G; ++g) {
    if (sizes[g] < 0) return fail(MX_ESHAPE, "%s: group %d has negative size", who, g);
    sum += sizes[g];
    sumP += pad32(sizes[g]);
  }
  if (mode == MX_GROUP_M && sum != M) return fail(MX_ESHAPE, "%s: sizes sum to %lld, expected M=%lld", who, (long long)sum, (long long)M);
  if (mode == MX_GROUP_K && sumP != K) return fail(MX_ESHAPE, "%s: padded sizes sum to %lld, expected K=%lld", who, (long long)sumP, (long long)K);
  if (mode == MX_GROUP_K && c_group_stride < 0) return fail(MX_ESHAPE, "%s: negative c_group_stride", who);

  GemmPlan& p = *plan;
  memset(&p.args, 0, sizeof(p.args));
  mx::GemmArgs& A = p.args;
  A.a = a; A.as = as; A.b = b; A.bs = bs; A.c = c;
  A.lda = lda; A.ldb = ldb; A.ldc = ldc;
  A.b_group_stride = b_group_stride;
  A.bs_group_stride = b_group_stride / 32;
  A.sa = mx::row_major_scales(lda);
  A.sb = mx::row_major_scales(ldb);
  A.as_bytes = M * (lda / 32);
  // extent of the B scale array: up to the last valid scale of the last row
  // of the last group in group-M (row r of group g spans K codes from
  // g * b_group_stride + r * ldb), B itself in group-K
  A.bs_bytes = mode == MX_GROUP_M ? ((int64_t)(G - 1) * b_group_stride + (n_rows_b - 1) * ldb + K) / 32
                                  : n_rows_b * (ldb / 32);
  A.c_group_stride = c_group_stride;
  A.M = (int32_t)M; A.N = (int32_t)N; A.K = (int32_t)K;
  A.accumulate = accumulate;
  const int64_t tiles_n = epi == mx::EPI_SWIGLU_FWD ? cdiv(N / 2, mx::kTileN / 2) : cdiv(N, mx::kTileN);
  A.n_tiles_n = (int32_t)tiles_n;
  // slot order: group-M keeps expert order and drops empty groups; group-K puts
  // the longest contractions first so the tail of the launch is short.
  std::vector<int> order;
  for (int g = 0; g < G; ++g)
    if (mode == MX_GROUP_K || sizes[g] > 0) order.push_back(g);
  if (mode == MX_GROUP_K)
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return sizes[x] > sizes[y]; });
  std::vector<int64_t> r0(G + 1, 0), p0(G + 1, 0);
  for (int g = 0; g < G; ++g) { r0[g + 1] = r0[g] + sizes[g]; p0[g + 1] = p0[g] + pad32(sizes[g]); }
  int64_t t = 0;
  A.groups.n = (int32_t)order.size();
  for (size_t s = 0; s < order.size(); ++s) {
    const int g = order[s];
    A.groups.tile0[s] = (int32_t)t;
    A.groups.gid[s] = g;
    A.groups.pc0[s] = (int32_t)p0[g];
    if (mode == MX_GROUP_M) {
      A.groups.a0[s] = (int32_t)r0[g];
      A.groups.len[s] = (int32_t)sizes[g];
      t += cdiv(sizes[g], mx::kTileM) * tiles_n;
    } else {
      A.groups.a0[s] = (int32_t)p0[g];
      A.groups.len[s] = (int32_t)pad32(sizes[g]);
      t += cdiv(M, mx::kTileM) * tiles_n;
    }
  }
  A.groups.tile0[order.size()] = (int32_t)t;
  if (t > kI32Max) return fail(MX_EUNSUPPORTED, "%s: too many tiles", who);
  // group-K: every slot has cdiv(M, 256) * tiles_n tiles; when that is a
  // whole number of 32-tile XCD chunks the kernel interleaves the slots
  const int64_t per_slot = cdiv(M, mx::kTileM) * tiles_n;
  A.groups.interleave = mode == MX_GROUP_K && order.size() > 1 && per_slot % 32 == 0 ? 1 : 0;
  p.total_tiles = (int)t;
  // whole-dword scale loads: every k tile starts at a multiple of 4 blocks
  p.scale_dword = mode == MX_GROUP_M && K % 128 == 0 && lda % 128 == 0 && ldb % 128 == 0 &&
                  b_group_stride % 128 == 0 && aligned(as, 4) && aligned(bs, 4);
  if (M == 0 || (mode == MX_GROUP_M && sum == 0)) p.total_tiles = 0;
  return MX_OK;
}

// Switch a plan of the fused MLP to its k-tiled scale buffers: A scales of
// a_rows rows with nq_a steps, B scales of b_rows rows (all groups) with nq_b
// steps, B group g's scales bs_group_stride bytes after group g-1's, and the
// activation layout's per-expert first steps (group-K contraction steps and
// the columnwise epilogue outputs).
void use_k_tiled_scales(GemmPlan& p, int64_t nq_a, int64_t a_rows, int64_t nq_b, int64_t b_rows,
                        int64_t bs_group_stride, const std::vector<int64_t>& q0_act) {
  mx::GemmArgs& A = p.args;
  A.sa = mx::k_tiled_scales(nq_a);
  A.sb = mx::k_tiled_scales(nq_b);
  A.as_bytes = cdiv(a_rows, 32) * nq_a * 128;
  A.bs_bytes = cdiv(b_rows, 32) * nq_b * 128;
  A.bs_group_stride = bs_group_stride;
  A.k_tiled = 1;
  for (int s = 0; s < A.groups.n; ++s) A.groups.q0[s] = (int32_t)q0_act[A.groups.gid[s]];
  p.scale_dword = true;
}

// Number of compute units of the current device (cached per device).
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Split-K tail of a plain group-M plan: when the last round of tiles would
// leave at least half of the CUs idle, each tail tile's k-steps are split
// into parts that run as separate workgroups, writing fp32 partials to ws;
// launch_split_reduce then forms C. Returns the number of tail tiles (0: no
// split; the plan is unchanged).
size_t split_ws_bytes(int64_t tiles) { return (size_t)std::min<int64_t>(tiles, mx::kMaxSplitTiles) * mx::kMaxSplitParts * mx::kTileM * mx::kTileN * 4; }

int plan_split_tail(GemmPlan& p, int64_t K, float* ws, size_t ws_bytes) {
  const int n_cu = device_cu_count();
  const int T = p.total_tiles;
  if (n_cu <= 0 || T == 0 || K % mx::kTileK) return 0;
  const int F = T / n_cu * n_cu, R = T - F;
  if (R == 0 || R > n_cu / 2 || R > mx::kMaxSplitTiles) return 0;
  const int nk = (int)(K / mx::kTileK);
  const int S = std::min({mx::kMaxSplitParts, n_cu / R, nk / 4});
  if (S < 2 || (size_t)R * S * mx::kTileM * mx::kTileN * 4 > ws_bytes) return 0;
  p.args.split_f = F;
  p.args.split_s = S;
  p.args.split_ws = ws;
  p.total_tiles = F + R * S;
  return R;
}

// ---------------------------------------------------------------- fused MLP plan
struct MlpLayout {
  int E;
  int64_t R, H, F, sumP;
  std::vector<int64_t> split;
  // forward workspace
  size_t xq, xs, w1q, w1s, w2q, w2s, aq, as, split2, fwd_total;
  // saved for backward
  size_t xcq, xcs, h1, acq, acs, w1cq, w1cs, w2cq, w2cs, saved_total;
  // backward workspace
  size_t dyq, dys, dycq, dycs, dhq, dhs, dhcq, dhcs, part, split1, bwd_total;
  size_t split2_bytes, split1_bytes;   // split-K tail partials of GEMM2 / dgrad1
  int64_t n_tiles_f;
  std::vector<int64_t> q0;   // k-tiled steps of the per-expert columnwise layouts
  int64_t nq;                // total steps (q0[E])
  // device-resident split sizes: the layout holds every split of R rows
  // (split above is a placeholder that passes the host checks), the group
  // tables are built by the call's first kernel into plan_fwd / plan_bwd
  bool dev = false;
  const int64_t* counts_dev = nullptr;
  size_t plan_fwd = 0, plan_bwd = 0;
};

// Worst-case sums over any split of R rows into E groups (at most min(E, R)
// of them non-empty): sum of ceil(m_g / b) <= floor((R + (b-1) * min(E, R)) / b).
int64_t worst_blocks(int64_t R, int64_t E, int64_t b) { return (R + (b - 1) * std::min(E, R)) / b; }

size_t take(size_t& cur, size_t bytes) {
  const size_t at = cur;
  cur += (bytes + 255) / 256 * 256;
  return at;
}

mx_status mlp_layout(const mx_mlp_dims* d, const int64_t* split, MlpLayout* L, const char* who,
                     bool device_split = false) {
  if (!d) return fail(MX_EINVAL, "%s: dims is null", who);
  if (d->num_experts < 1) return fail(MX_EINVAL, "%s: need at least one expert", who);
  if (d->num_experts > mx::kMaxGroups) return fail(MX_EUNSUPPORTED, "%s: %d experts exceeds the maximum %d", who, d->num_experts, mx::kMaxGroups);
  std::vector<int64_t> placeholder;
  if (device_split) {
    placeholder.assign(d->num_experts, 0);
    placeholder[0] = d->rows > 0 ? d->rows : 0;
    split = placeholder.data();
  }
  if (!split) return fail(MX_EINVAL, "%s: split_sizes is null", who);
  if (d->rows < 0 || d->hidden <= 0 || d->ffn <= 0) return fail(MX_ESHAPE, "%s: bad dims", who);
  if (d->hidden % 128 || d->ffn % 128) return fail(MX_ESHAPE, "%s: hidden and ffn must be multiples of 128", who);
  if (d->rows > kI32Max || 2 * d->ffn > kI32Max || (int64_t)d->num_experts * 2 * d->ffn > kI32Max ||
      (int64_t)d->num_experts * d->hidden > kI32Max)
    return fail(MX_EUNSUPPORTED, "%s: dimensions exceed 2^31-1", who);
  mx_status st = check_groups(split, d->num_experts, d->rows, who);
  if (st != MX_OK) return st;
  L->E = d->num_experts;
  L->R = d->rows;
  L->H = d->hidden;
  L->F = d->ffn;
  L->split.assign(split, split + d->num_experts);
  L->sumP = 0;
  for (int e = 0; e < L->E; ++e) L->sumP += pad32(split[e]);
  L->q0 = group_steps(split, d->num_experts, d->rows);
  L->nq = L->q0[L->E];
  L->dev = device_split;
  if (device_split) {
    L->sumP = worst_blocks(L->R, L->E, 32) * 32;
    L->nq = worst_blocks(L->R, L->E, 128);
    if (worst_blocks(L->R, L->E, mx::kTileM) * cdiv(L->H, mx::kTileN) > kI32Max ||
        worst_blocks(L->R, L->E, mx::kQuantTileRows) * (L->H / 128) > kI32Max || L->sumP > kI32Max)
      return fail(MX_EUNSUPPORTED, "%s: too many tiles", who);
  }
  const int64_t R = L->R, H = L->H, F = L->F, E = L->E, P = L->sumP;
  // all scales are k-tiled: a rowwise [rows, K] matrix takes ceil(rows/32)*32*K/32
  // bytes, a per-expert columnwise [cols, P] one cols/32 * nq * 128
  const int64_t R32 = cdiv(R, 32) * 32, NQ = L->nq;
  size_t c = 0;
  L->xq = take(c, R * H); L->xs = take(c, R32 * H / 32);
  L->w1q = take(c, E * 2 * F * H); L->w1s = take(c, E * 2 * F * H / 32);
  L->w2q = take(c, E * H * F); L->w2s = take(c, E * H * F / 32);
  L->aq = take(c, R * F); L->as = take(c, R32 * F / 32);
  // GEMM2 and dgrad1 tiles: sum over experts of ceil(m_e/256) x ceil(H/256)
  int64_t m_tiles = 0;
  for (int e = 0; e < L->E; ++e) m_tiles += cdiv(split[e], mx::kTileM);
  const int64_t h_tiles = m_tiles * cdiv(H, mx::kTileN);
  // (no split-K tail with device-built tables: its plan needs the tile count)
  L->split2_bytes = L->split1_bytes = device_split ? 0 : split_ws_bytes(h_tiles);
  L->split2 = take(c, L->split2_bytes);
  if (device_split) L->plan_fwd = take(c, sizeof(mx::MlpDevPlan));
  L->fwd_total = c;
  c = 0;
  L->xcq = take(c, H * P); L->xcs = take(c, H / 32 * NQ * 128);
  L->h1 = take(c, R * 2 * F * 2);
  L->acq = take(c, F * P); L->acs = take(c, F / 32 * NQ * 128);
  L->w1cq = take(c, H * E * 2 * F); L->w1cs = take(c, H * E * 2 * F / 32);
  L->w2cq = take(c, F * E * H); L->w2cs = take(c, F * E * H / 32);
  L->saved_total = c;
  c = 0;
  L->n_tiles_f = cdiv(F, mx::kTileN);
  L->dyq = take(c, R * H); L->dys = take(c, R32 * H / 32);
  L->dycq = take(c, H * P); L->dycs = take(c, H / 32 * NQ * 128);
  L->dhq = take(c, R * 2 * F); L->dhs = take(c, R32 * 2 * F / 32);
  L->dhcq = take(c, 2 * F * P); L->dhcs = take(c, 2 * F / 32 * NQ * 128);
  L->part = take(c, L->n_tiles_f * R * 4);
  L->split1 = take(c, L->split1_bytes);
  if (device_split) L->plan_bwd = take(c, sizeof(mx::MlpDevPlan));
  L->bwd_total = c;
  return MX_OK;
}

uint8_t* at(void* base, size_t off) { return reinterpret_cast<uint8_t*>(base) + off; }
const uint8_t* at(const void* base, size_t off) { return reinterpret_cast<const uint8_t*>(base) + off; }

// MXFP8 copies of the expert weights, both layouts with k-tiled scales:
// W1 rowwise [E*2F, H], W2 rowwise [E*H, F], W1 columnwise [H, E*2F] (groups
// of 2F columns per expert) and W2 columnwise [F, E*H] (groups of H).
struct WeightCopies {
  uint8_t *w1q, *w1s, *w2q, *w2s;      // rowwise (forward GEMMs)
  uint8_t *w1cq, *w1cs, *w2cq, *w2cs;  // columnwise (dgrad GEMMs)
};

// Layout of a weight cache buffer (grouped_mlp_quantize_weights): the four
// copies back to back, 256-byte aligned regions; offsets depend on E, H, F only.
struct WeightCacheLayout {
  size_t w1q, w1s, w2q, w2s, w1cq, w1cs, w2cq, w2cs, total;
};

WeightCacheLayout weight_cache_layout(int64_t E, int64_t H, int64_t F) {
  WeightCacheLayout W;
  size_t c = 0;
  W.w1q = take(c, E * 2 * F * H); W.w1s = take(c, E * 2 * F * H / 32);
  W.w2q = take(c, E * H * F); W.w2s = take(c, E * H * F / 32);
  W.w1cq = take(c, H * E * 2 * F); W.w1cs = take(c, H * E * 2 * F / 32);
  W.w2cq = take(c, F * E * H); W.w2cs = take(c, F * E * H / 32);
  W.total = c;
  return W;
}

WeightCopies weight_cache_copies(const WeightCacheLayout& W, void* base) {
  return {at(base, W.w1q), at(base, W.w1s), at(base, W.w2q), at(base, W.w2s),
          at(base, W.w1cq), at(base, W.w1cs), at(base, W.w2cq), at(base, W.w2cs)};
}

// Quantize the bf16 master weights into both MXFP8 layouts (columnwise
// copies skipped where their pointers are null).
mx_status quantize_weights_into(const MlpLayout& L, const void* w1, const void* w2, const WeightCopies& wc,
                                hipStream_t stream, bool marks) {
  const int64_t H = L.H, F = L.F;
  const int E = L.E;
  std::vector<int64_t> g_w1(E, 2 * F), g_w2(E, H);
  if (marks) stage_mark(1, stream);
  mx_status st = quantize_impl(w1, MX_BF16, E * 2 * F, H, g_w1.data(), E, wc.w1q, wc.w1s, wc.w1cq, wc.w1cs,
                               stream, true);
  if (st != MX_OK) return st;
  if (marks) stage_mark(2, stream);
  return quantize_impl(w2, MX_BF16, E * H, F, g_w2.data(), E, wc.w2q, wc.w2s, wc.w2cq, wc.w2cs, stream, true);
}

// Device-built group tables (device-resident split sizes): tile counts of
// the tables in mx::MlpDevPlan, from the dims alone.
enum : int { kDevGemm1 = 0, kDevNH = 1, kDevNF = 2 };     // group-M tables
enum : int { kDevWgrad2 = 0, kDevWgrad1 = 1 };            // group-K tables

mx::MlpDevPlanArgs dev_plan_args(const MlpLayout& L, mx::MlpDevPlan* plan) {
  mx::MlpDevPlanArgs a;
  memset(&a, 0, sizeof(a));
  a.counts = L.counts_dev;
  a.plan = plan;
  a.E = L.E;
  a.R = (int32_t)L.R;
  a.m_tiles_n[kDevGemm1] = (int32_t)cdiv(L.F, mx::kTileN / 2);
  a.m_tiles_n[kDevNH] = (int32_t)cdiv(L.H, mx::kTileN);
  a.m_tiles_n[kDevNF] = (int32_t)cdiv(L.F, mx::kTileN);
  a.k_slot_tiles[kDevWgrad2] = (int32_t)(cdiv(L.H, mx::kTileM) * cdiv(L.F, mx::kTileN));
  a.k_slot_tiles[kDevWgrad1] = (int32_t)(cdiv(2 * L.F, mx::kTileM) * cdiv(L.H, mx::kTileN));
  for (int j = 0; j < 2; ++j) a.k_interleave[j] = L.E > 1 && a.k_slot_tiles[j] % 32 == 0 ? 1 : 0;
  return a;
}

// Switch a plan built on the placeholder split to device table j of plan:
// worst-case grid, no split-K tail. The table's tile counts must be the
// plan's own (an internal consistency check).
mx_status use_dev_groups(GemmPlan& p, int mode, const MlpLayout& L, mx::MlpDevPlan* plan, int j) {
  const mx::MlpDevPlanArgs a = dev_plan_args(L, plan);
  mx::GemmArgs& A = p.args;
  int64_t worst;
  if (mode == MX_GROUP_M) {
    if (A.n_tiles_n != a.m_tiles_n[j]) return fail(MX_EUNSUPPORTED, "internal: device table %d tile count", j);
    A.groups_dev = &plan->m[j];
    worst = worst_blocks(L.R, L.E, mx::kTileM) * A.n_tiles_n;
  } else {
    if (cdiv(A.M, mx::kTileM) * A.n_tiles_n != a.k_slot_tiles[j] || A.groups.interleave != a.k_interleave[j])
      return fail(MX_EUNSUPPORTED, "internal: device table %d tile count", j);
    A.groups_dev = &plan->k[j];
    worst = (int64_t)L.E * a.k_slot_tiles[j];
  }
  A.split_s = 0;
  p.total_tiles = (int)worst;
  return MX_OK;
}

mx_status run_gemm(const GemmPlan& p, int mode, int epi, hipStream_t stream, const char* what) {
  hipError_t e = mx::launch_gemm(mode, epi, p.scale_dword, p.args, p.total_tiles, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return MX_OK;
}

}  // namespace

// 4-bit (grouped) GEMM, MXFP4 or (nv) NVFP4 operands: validation, group
// table, launch.
// split_ws (MXFP4 only; may be null): room for the fp32 partials of a
// split-K tail, planned as for the MXFP8 GEMMs (plan_split_tail) with the
// 4-bit kernel's 256-value k-tiles.
static mx_status gemm_4bit_impl(const char* who, bool nv, const uint8_t* a, const uint8_t* a_s, const float* a_amax,
                                const uint8_t* b, const uint8_t* b_s, const float* b_amax, const int64_t* sizes,
                                int32_t groups, int64_t n, int64_t k, void* c, mx_dtype c_dtype, void* stream,
                                float* split_ws = nullptr, size_t split_ws_bytes = 0) {
  if (c_dtype != MX_BF16 && c_dtype != MX_F32) return fail(MX_EINVAL, "%s: bad output dtype", who);
  if (groups < 1 || groups > MX_MAX_GROUPS) return fail(MX_EINVAL, "%s: need 1 <= groups <= %d", who, MX_MAX_GROUPS);
  if (!sizes) return fail(MX_EINVAL, "%s: null group sizes", who);
  const int64_t kq = nv ? 128 : 64;
  if (n < 0 || k <= 0 || k % kq)
    return fail(MX_ESHAPE, "%s: need n >= 0 and k a positive multiple of %lld", who, (long long)kq);
  if (k > ((int64_t)1 << 24)) return fail(MX_EUNSUPPORTED, "%s: k above 2^24", who);
  mx::Fp4Groups gr{};
  gr.n = groups;
  int64_t rows = 0, mtiles = 0;
  for (int g = 0; g < groups; ++g) {
    if (sizes[g] < 0) return fail(MX_ESHAPE, "%s: negative group size", who);
    gr.row0[g] = rows;
    gr.tile0[g] = (int32_t)(mtiles < kI32Max ? mtiles : kI32Max);
    rows += sizes[g];
    mtiles += (sizes[g] + mx::kFp4GemmTileM - 1) / mx::kFp4GemmTileM;
  }
  gr.row0[groups] = rows;
  const int64_t ntiles = (n + mx::kFp4GemmTileN - 1) / mx::kFp4GemmTileN;
  if (mtiles * ntiles > kI32Max) return fail(MX_EUNSUPPORTED, "%s: too many output tiles", who);
  gr.tile0[groups] = (int32_t)mtiles;
  if (rows == 0 || n == 0) return MX_OK;
  if (!a || !a_s || !b || !b_s || !c || (nv && (!a_amax || !b_amax)))
    return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16))
    return fail(MX_EALIGN, "%s: a, b and c must be 16-byte aligned", who);
  if (nv && (!aligned(a_s, 8) || !aligned(b_s, 8) || !aligned(a_amax, 4) || !aligned(b_amax, 4)))
    return fail(MX_EALIGN, "%s: scales must be 8-byte and tensor amax 4-byte aligned", who);
  mx::Fp4Split sp{0, 0, nullptr};
  if (!nv && split_ws != nullptr) {
    const int n_cu = device_cu_count();
    const int64_t T = mtiles * ntiles;
    const int64_t full = n_cu > 0 ? T / n_cu * n_cu : T, tail = T - full;
    const int64_t nk = (k + 255) / 256;
    if (n_cu > 0 && tail > 0 && tail <= n_cu / 2 && tail <= mx::kMaxSplitTiles) {
      const int64_t parts = std::min<int64_t>({mx::kMaxSplitParts, n_cu / tail, nk / 4});
      if (parts >= 2 && (size_t)(tail * parts) * mx::kFp4GemmTileM * mx::kFp4GemmTileN * 4 <= split_ws_bytes)
        sp = mx::Fp4Split{(int32_t)full, (int32_t)parts, split_ws};
    }
  }
  hipError_t e = nv ? mx::launch_gemm_nvfp4(a, a_s, a_amax, b, b_s, b_amax, gr, n, k, c, c_dtype == MX_F32 ? 1 : 0,
                                            reinterpret_cast<hipStream_t>(stream))
                    : mx::launch_gemm_fp4(a, a_s, b, b_s, gr, n, k, c, c_dtype == MX_F32 ? 1 : 0,
                                          reinterpret_cast<hipStream_t>(stream), sp);
  if (e != hipSuccess) return hip_fail(e, who);
  return MX_OK;
}

static mx_status gemm_fp4_impl(const char* who, const uint8_t* a, const uint8_t* a_s, const uint8_t* b,
                               const uint8_t* b_s, const int64_t* sizes, int32_t groups, int64_t n, int64_t k,
                               void* c, mx_dtype c_dtype, void* stream, float* split_ws = nullptr,
                               size_t split_ws_bytes = 0) {
  return gemm_4bit_impl(who, false, a, a_s, nullptr, b, b_s, nullptr, sizes, groups, n, k, c, c_dtype, stream,
                        split_ws, split_ws_bytes);
}

extern "C" {

const char* mx_status_string(int s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_EINVAL: return "MX_EINVAL";
    case MX_ESHAPE: return "MX_ESHAPE";
    case MX_EALIGN: return "MX_EALIGN";
    case MX_EWORKSPACE: return "MX_EWORKSPACE";
    case MX_EHIP: return "MX_EHIP";
    case MX_EUNSUPPORTED: return "MX_EUNSUPPORTED";
    default: return "MX_UNKNOWN";
  }
}

const char* mx_last_error(void) { return g_err; }

mx_status mx_set_stage_events(void* const* events, int32_t count) {
  g_err[0] = 0;
  if (count < 0 || (count > 0 && events == nullptr))
    return fail(MX_EINVAL, "mx_set_stage_events: bad event array");
  g_events = count > 0 ? events : nullptr;
  g_n_events = count;
  return MX_OK;
}

int mx_version(void) { return 1; }

mx_status mx_device_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_device_copy";
  if (bytes < 0 || bytes % 16) return fail(MX_ESHAPE, "%s: bytes must be a non-negative multiple of 16", who);
  if (bytes > 0 && (!dst || !src)) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(dst, 16) || !aligned(src, 16)) return fail(MX_EALIGN, "%s: dst and src must be 16-byte aligned", who);
  hipError_t e = mx::launch_device_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_device_copy launch");
  return MX_OK;
}

mx_status mx_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const int64_t* group_sizes,
                      int32_t num_groups, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                      void* stream) {
  g_err[0] = 0;
  return quantize_impl(x, x_dtype, rows, cols, group_sizes, num_groups, q_row, s_row, q_col, s_col,
                       reinterpret_cast<hipStream_t>(stream));
}

mx_status mx_grouped_gemm(int32_t mode, int32_t num_groups, const int64_t* sizes, int64_t M, int64_t N, int64_t K,
                          const uint8_t* a, const uint8_t* a_scale, int64_t lda, const uint8_t* b,
                          const uint8_t* b_scale, int64_t ldb, int64_t b_group_stride, void* c, int32_t c_dtype,
                          int64_t ldc, int64_t c_group_stride, int32_t accumulate, void* stream) {
  g_err[0] = 0;
  GemmPlan p;
  const int epi = c_dtype == MX_BF16 ? mx::EPI_BF16 : mx::EPI_F32;
  mx_status st = gemm_plan(mode, num_groups, sizes, M, N, K, a, a_scale, lda, b, b_scale, ldb, b_group_stride, c,
                           c_dtype, ldc, c_group_stride, accumulate, epi, N, &p);
  if (st != MX_OK) return st;
  return run_gemm(p, mode, epi, reinterpret_cast<hipStream_t>(stream), "mx_grouped_gemm launch");
}

mx_status grouped_mlp_sizes(const mx_mlp_dims* dims, const int64_t* split_sizes, size_t* fwd_workspace,
                            size_t* saved, size_t* bwd_workspace) {
  g_err[0] = 0;
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, "grouped_mlp_sizes");
  if (st != MX_OK) return st;
  if (fwd_workspace) *fwd_workspace = L.fwd_total;
  if (saved) *saved = L.saved_total;
  if (bwd_workspace) *bwd_workspace = L.bwd_total;
  return MX_OK;
}

mx_status grouped_mlp_intermediates(const mx_mlp_dims* dims, const int64_t* split_sizes, mx_mlp_intermediates* out) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_intermediates";
  if (!out) return fail(MX_EINVAL, "%s: out is null", who);
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  out->a_row_codes = L.aq;
  out->a_row_scales = L.as;
  out->h1 = L.h1;
  out->a_col_codes = L.acq;
  out->a_col_scales = L.acs;
  out->dh1_row_codes = L.dhq;
  out->dh1_row_scales = L.dhs;
  out->dh1_col_codes = L.dhcq;
  out->dh1_col_scales = L.dhcs;
  out->nq_col = L.nq;
  return MX_OK;
}

}  // extern "C"

namespace {

// The fused forward after argument checks. With wc_cached null the weights
// are cast from w1/w2 into the workspace (rowwise) and saved (columnwise)
// copies; otherwise the cached copies are used and w1/w2 are not read.
mx_status fwd_impl(const MlpLayout& L, const void* x, const float* probs, const void* w1, const void* w2,
                   const WeightCopies* wc_cached, void* y, void* saved, void* workspace, hipStream_t stream,
                   const int32_t* row_token = nullptr, int64_t tokens = 0) {
  const int64_t R = L.R, H = L.H, F = L.F;
  const int E = L.E;
  const WeightCopies wc = wc_cached ? *wc_cached
      : WeightCopies{at(workspace, L.w1q), at(workspace, L.w1s), at(workspace, L.w2q), at(workspace, L.w2s),
                     saved ? at(saved, L.w1cq) : nullptr, saved ? at(saved, L.w1cs) : nullptr,
                     saved ? at(saved, L.w2cq) : nullptr, saved ? at(saved, L.w2cs) : nullptr};
  // plan both GEMMs before launching anything
  GemmPlan p1, p2;
  mx_status st = gemm_plan(MX_GROUP_M, E, L.split.data(), R, 2 * F, H, at(workspace, L.xq), at(workspace, L.xs), H,
                           wc.w1q, wc.w1s, H, 2 * F * H, y, MX_BF16, 2 * F, 0, 0, mx::EPI_SWIGLU_FWD, 2 * F, &p1);
  if (st != MX_OK) return st;
  st = gemm_plan(MX_GROUP_M, E, L.split.data(), R, H, F, at(workspace, L.aq), at(workspace, L.as), F,
                 wc.w2q, wc.w2s, F, H * F, y, MX_BF16, H, 0, 0, mx::EPI_BF16, H, &p2);
  if (st != MX_OK) return st;
  use_k_tiled_scales(p1, H / 128, R, H / 128, E * 2 * F, 2 * F * H / 32, L.q0);
  use_k_tiled_scales(p2, F / 128, R, F / 128, E * H, H * F / 32, L.q0);
  mx::GemmArgs& a1 = p1.args;
  a1.c = nullptr;
  a1.nq_row = (int32_t)(F / 128);
  a1.nq_col = (int32_t)L.nq;
  a1.F = (int32_t)F;
  a1.ld_col = L.sumP;
  a1.probs = probs;
  a1.h1 = saved ? reinterpret_cast<uint16_t*>(at(saved, L.h1)) : nullptr;
  a1.q_row = at(workspace, L.aq);
  a1.s_row = at(workspace, L.as);
  a1.q_col = saved ? at(saved, L.acq) : nullptr;
  a1.s_col = saved ? at(saved, L.acs) : nullptr;
  a1.R = (int32_t)R;
  mx::MlpDevPlan* plan = L.dev ? reinterpret_cast<mx::MlpDevPlan*>(at(workspace, L.plan_fwd)) : nullptr;
  DevQuant dq{};
  if (L.dev) {
    st = use_dev_groups(p1, MX_GROUP_M, L, plan, kDevGemm1);
    if (st == MX_OK) st = use_dev_groups(p2, MX_GROUP_M, L, plan, kDevNH);
    if (st != MX_OK) return st;
    dq = DevQuant{&plan->act, L.sumP, (int32_t)L.nq, worst_blocks(R, E, mx::kQuantTileRows)};
  }

  stage_mark(0, stream);
  if (L.dev) {
    hipError_t e = mx::launch_mlp_dev_plan(dev_plan_args(L, plan), stream);
    if (e != hipSuccess) return hip_fail(e, "grouped_mlp_fwd device plan");
  }
  // (with row_token: routed row r is token row row_token[r] of x, gathered
  // by the cast itself)
  st = quantize_impl(x, MX_BF16, R, H, L.split.data(), E, at(workspace, L.xq), at(workspace, L.xs),
                     saved ? at(saved, L.xcq) : nullptr, saved ? at(saved, L.xcs) : nullptr, stream, true,
                     row_token, tokens, L.dev ? &dq : nullptr);
  if (st != MX_OK) return st;
  // (running the W2 cast on the side stream beside GEMM1 was measured: it
  // slows GEMM1 by more than the cast takes, so the forward stays serial)
  if (wc_cached) {
    stage_mark(1, stream);      // the weight stages are empty
    stage_mark(2, stream);
  } else {
    st = quantize_weights_into(L, w1, w2, wc, stream, true);
    if (st != MX_OK) return st;
  }
  stage_mark(3, stream);
  st = run_gemm(p1, MX_GROUP_M, mx::EPI_SWIGLU_FWD, stream, "grouped_mlp_fwd gemm1");
  if (st != MX_OK) return st;
  stage_mark(4, stream);
  {
    const int tail = L.dev ? 0 : plan_split_tail(p2, F, reinterpret_cast<float*>(at(workspace, L.split2)),
                                                 L.split2_bytes);
    st = run_gemm(p2, MX_GROUP_M, mx::EPI_BF16, stream, "grouped_mlp_fwd gemm2");
    if (st != MX_OK) return st;
    hipError_t e = mx::launch_split_reduce(mx::EPI_BF16, p2.args, tail, stream);
    if (e != hipSuccess) return hip_fail(e, "grouped_mlp_fwd gemm2 split reduce");
  }
  stage_mark(5, stream);
  return MX_OK;
}

mx_status fwd_checks(const MlpLayout& L, const void* x, const float* probs, const void* y, const void* saved,
                     size_t saved_bytes, const void* workspace, size_t workspace_bytes, const char* who) {
  if (!x || !y || !workspace) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256) || (saved && !aligned(saved, 256)) ||
      (probs && !aligned(probs, 4)))
    return fail(MX_EALIGN, "%s: x, y must be 16-byte and workspace/saved 256-byte aligned", who);
  if (workspace_bytes < L.fwd_total)
    return fail(MX_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, L.fwd_total);
  if (saved && saved_bytes < L.saved_total)
    return fail(MX_EWORKSPACE, "%s: saved buffer %zu bytes < required %zu", who, saved_bytes, L.saved_total);
  return MX_OK;
}

mx_status cache_checks(const MlpLayout& L, const void* cache, size_t cache_bytes, WeightCacheLayout* W,
                       const char* who) {
  *W = weight_cache_layout(L.E, L.H, L.F);
  if (!cache) return fail(MX_EINVAL, "%s: weight cache is null", who);
  if (!aligned(cache, 256)) return fail(MX_EALIGN, "%s: weight cache must be 256-byte aligned", who);
  if (cache_bytes < W->total)
    return fail(MX_EWORKSPACE, "%s: weight cache %zu bytes < required %zu", who, cache_bytes, W->total);
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status grouped_mlp_fwd(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* x, const float* probs,
                          const void* w1, const void* w2, void* y, void* saved, size_t saved_bytes,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fwd_checks(L, x, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  if (!w1 || !w2) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte aligned", who);
  return fwd_impl(L, x, probs, w1, w2, nullptr, y, saved, workspace, reinterpret_cast<hipStream_t>(stream));
}

mx_status grouped_mlp_fwd_gather(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* x_tokens,
                                 int64_t tokens, const int32_t* row_token, const float* probs, const void* w1,
                                 const void* w2, void* y, void* saved, size_t saved_bytes, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd_gather";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fwd_checks(L, x_tokens, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  if (!w1 || !w2 || (L.R > 0 && !row_token)) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (tokens < 0 || tokens > kI32Max) return fail(MX_ESHAPE, "%s: bad token count %lld", who, (long long)tokens);
  if (!aligned(w1, 16) || !aligned(w2, 16) || !aligned(row_token, 4))
    return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte and row_token 4-byte aligned", who);
  return fwd_impl(L, x_tokens, probs, w1, w2, nullptr, y, saved, workspace, reinterpret_cast<hipStream_t>(stream),
                  row_token, tokens);
}

mx_status grouped_mlp_weight_cache_bytes(const mx_mlp_dims* dims, size_t* bytes) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_weight_cache_bytes";
  if (!bytes) return fail(MX_EINVAL, "%s: bytes is null", who);
  if (!dims) return fail(MX_EINVAL, "%s: dims is null", who);
  // the cache does not depend on the routed rows: check the rest with R = 0
  mx_mlp_dims d = *dims;
  d.rows = 0;
  std::vector<int64_t> zeros(d.num_experts > 0 && d.num_experts <= mx::kMaxGroups ? d.num_experts : 1, 0);
  MlpLayout L;
  mx_status st = mlp_layout(&d, zeros.data(), &L, who);
  if (st != MX_OK) return st;
  *bytes = weight_cache_layout(L.E, L.H, L.F).total;
  return MX_OK;
}

mx_status grouped_mlp_quantize_weights(const mx_mlp_dims* dims, const void* w1, const void* w2, void* cache,
                                       size_t cache_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_quantize_weights";
  if (!dims) return fail(MX_EINVAL, "%s: dims is null", who);
  mx_mlp_dims d = *dims;
  d.rows = 0;
  std::vector<int64_t> zeros(d.num_experts > 0 && d.num_experts <= mx::kMaxGroups ? d.num_experts : 1, 0);
  MlpLayout L;
  mx_status st = mlp_layout(&d, zeros.data(), &L, who);
  if (st != MX_OK) return st;
  WeightCacheLayout W;
  st = cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  if (!w1 || !w2) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte aligned", who);
  return quantize_weights_into(L, w1, w2, weight_cache_copies(W, cache), reinterpret_cast<hipStream_t>(stream),
                               false);
}

mx_status grouped_mlp_fwd_cached(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* x,
                                 const float* probs, const void* cache, size_t cache_bytes, void* y, void* saved,
                                 size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd_cached";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fwd_checks(L, x, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  WeightCacheLayout W;
  st = cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  const WeightCopies wc = weight_cache_copies(W, const_cast<void*>(cache));
  return fwd_impl(L, x, probs, nullptr, nullptr, &wc, y, saved, workspace, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

mx_status bwd_checks(const MlpLayout& L, const void* dy, const float* probs, const void* saved, size_t saved_bytes,
                     const void* dx, const float* dprobs, const float* dw1, const float* dw2, const void* workspace,
                     size_t workspace_bytes, const char* who) {
  if (!dy || !saved || !dx || !dw1 || !dw2 || !workspace) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw1, 16) || !aligned(dw2, 16) || !aligned(saved, 256) ||
      !aligned(workspace, 256) || (probs && !aligned(probs, 4)) || (dprobs && !aligned(dprobs, 4)))
    return fail(MX_EALIGN, "%s: dy, dx, dw1, dw2 must be 16-byte and saved/workspace 256-byte aligned", who);
  if (saved_bytes < L.saved_total)
    return fail(MX_EWORKSPACE, "%s: saved buffer %zu bytes < required %zu", who, saved_bytes, L.saved_total);
  if (workspace_bytes < L.bwd_total)
    return fail(MX_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, L.bwd_total);
  return MX_OK;
}

// The fused backward after argument checks; the columnwise weight copies
// come from saved (w1c/w2c null) or from a weight cache.
mx_status bwd_impl(const MlpLayout& L, const void* dy, const float* probs, const void* saved,
                   const WeightCopies* wc_cached, void* dx, float* dprobs, float* dw1, float* dw2,
                   int32_t accumulate_wgrad, void* workspace, hipStream_t stream,
                   const int32_t* row_token = nullptr, int64_t tokens = 0) {
  const int64_t R = L.R, H = L.H, F = L.F, P = L.sumP;
  const int E = L.E;
  const uint8_t* w1cq = wc_cached ? wc_cached->w1cq : at(saved, L.w1cq);
  const uint8_t* w1cs = wc_cached ? wc_cached->w1cs : at(saved, L.w1cs);
  const uint8_t* w2cq = wc_cached ? wc_cached->w2cq : at(saved, L.w2cq);
  const uint8_t* w2cs = wc_cached ? wc_cached->w2cs : at(saved, L.w2cs);
  GemmPlan pd2, pw2, pd1, pw1;
  // dA = dY_row . colwise(W2_e): B_e = w2 columnwise [F, E*H] at column e*H
  mx_status st = gemm_plan(MX_GROUP_M, E, L.split.data(), R, F, H, at(workspace, L.dyq), at(workspace, L.dys), H,
                           w2cq, w2cs, E * H, H, dx, MX_BF16, F, 0, 0, mx::EPI_SWIGLU_BWD, F, &pd2);
  if (st != MX_OK) return st;
  // dW2_e = colwise(dY_e) . colwise(A_e)^T
  // (the contraction of the group-K plans is the padded split; with device
  // split sizes the placeholder's, inside the worst-case pitch P)
  const int64_t Kk = L.dev ? pad32(R) : P;
  st = gemm_plan(MX_GROUP_K, E, L.split.data(), H, F, Kk, at(workspace, L.dycq), at(workspace, L.dycs), P,
                 at(saved, L.acq), at(saved, L.acs), P, 0, dw2, MX_F32, F, H * F, accumulate_wgrad, mx::EPI_F32, F, &pw2);
  if (st != MX_OK) return st;
  // dX = dH1_row . colwise(W1_e): B_e = w1 columnwise [H, E*2F] at column e*2F
  st = gemm_plan(MX_GROUP_M, E, L.split.data(), R, H, 2 * F, at(workspace, L.dhq), at(workspace, L.dhs), 2 * F,
                 w1cq, w1cs, E * 2 * F, 2 * F, dx, MX_BF16, H, 0, 0, mx::EPI_BF16, H, &pd1);
  if (st != MX_OK) return st;
  // dW1_e = colwise(dH1_e) . colwise(X_e)^T
  st = gemm_plan(MX_GROUP_K, E, L.split.data(), 2 * F, H, Kk, at(workspace, L.dhcq), at(workspace, L.dhcs), P,
                 at(saved, L.xcq), at(saved, L.xcs), P, 0, dw1, MX_F32, H, 2 * F * H, accumulate_wgrad, mx::EPI_F32,
                 H, &pw1);
  if (st != MX_OK) return st;
  // B of dgrad2 / dgrad1: the columnwise weights [F, E*H] / [H, E*2F], expert
  // e's k range starting at step e*H/128 / e*2F/128
  use_k_tiled_scales(pd2, H / 128, R, E * H / 128, F, H, L.q0);
  use_k_tiled_scales(pw2, L.nq, H, L.nq, F, 0, L.q0);
  use_k_tiled_scales(pd1, 2 * F / 128, R, E * 2 * F / 128, H, 2 * F, L.q0);
  use_k_tiled_scales(pw1, L.nq, 2 * F, L.nq, H, 0, L.q0);
  mx::GemmArgs& a = pd2.args;
  a.c = nullptr;
  a.nq_row = (int32_t)(2 * F / 128);
  a.nq_col = (int32_t)L.nq;
  a.F = (int32_t)F;
  a.ld_col = P;
  a.probs = probs;
  a.h1 = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(at(saved, L.h1)));
  a.q_row = at(workspace, L.dhq);
  a.s_row = at(workspace, L.dhs);
  a.q_col = at(workspace, L.dhcq);
  a.s_col = at(workspace, L.dhcs);
  a.dprobs_part = dprobs ? reinterpret_cast<float*>(at(workspace, L.part)) : nullptr;
  a.R = (int32_t)R;
  mx::MlpDevPlan* plan = L.dev ? reinterpret_cast<mx::MlpDevPlan*>(at(workspace, L.plan_bwd)) : nullptr;
  DevQuant dq{};
  if (L.dev) {
    st = use_dev_groups(pd2, MX_GROUP_M, L, plan, kDevNF);
    if (st == MX_OK) st = use_dev_groups(pd1, MX_GROUP_M, L, plan, kDevNH);
    if (st == MX_OK) st = use_dev_groups(pw2, MX_GROUP_K, L, plan, kDevWgrad2);
    if (st == MX_OK) st = use_dev_groups(pw1, MX_GROUP_K, L, plan, kDevWgrad1);
    if (st != MX_OK) return st;
    dq = DevQuant{&plan->act, P, (int32_t)L.nq, worst_blocks(R, E, mx::kQuantTileRows)};
  }

  // stages overlap on the side stream unless per-stage timing is on: the
  // wgrad GEMMs (HBM-bound fp32 read-modify-write) run there, wgrad2 beside
  // dgrad2 and wgrad1 (which needs dH1 from dgrad2) beside dgrad1
  SideStream* sd = nullptr;
  if (g_events == nullptr) {
    st = side_stream(&sd);
    if (st != MX_OK) return st;
  }
  stage_mark(0, stream);
  if (L.dev) {
    hipError_t e = mx::launch_mlp_dev_plan(dev_plan_args(L, plan), stream);
    if (e != hipSuccess) return hip_fail(e, "grouped_mlp_bwd device plan");
  }
  // (with row_token: routed row r of dY is token row row_token[r] of dy)
  st = quantize_impl(dy, MX_BF16, R, H, L.split.data(), E, at(workspace, L.dyq), at(workspace, L.dys),
                     at(workspace, L.dycq), at(workspace, L.dycs), stream, true, row_token, tokens,
                     L.dev ? &dq : nullptr);
  if (st != MX_OK) return st;
  // once work is on the side stream, an error return still joins it first,
  // so nothing enqueued by this call runs unordered with the caller's stream
  auto fail_joined = [&](mx_status s) {
    if (sd != nullptr) {
      char keep[sizeof(g_err)];
      memcpy(keep, g_err, sizeof(g_err));
      (void)wait_for(stream, sd->s, sd->ev[2]);
      memcpy(g_err, keep, sizeof(g_err));
    }
    return s;
  };
  if (sd != nullptr) {
    st = wait_for(sd->s, stream, sd->ev[0]);
    if (st == MX_OK) st = run_gemm(pw2, MX_GROUP_K, mx::EPI_F32, sd->s, "grouped_mlp_bwd wgrad2");
    if (st != MX_OK) return fail_joined(st);
  }
  stage_mark(1, stream);
  st = run_gemm(pd2, MX_GROUP_M, mx::EPI_SWIGLU_BWD, stream, "grouped_mlp_bwd dgrad2");
  if (st != MX_OK) return fail_joined(st);
  stage_mark(2, stream);
  if (dprobs) {
    hipError_t e = mx::launch_dprobs_reduce(reinterpret_cast<const float*>(at(workspace, L.part)), dprobs,
                                            (int32_t)R, (int32_t)L.n_tiles_f, L.dev ? &plan->rows : nullptr,
                                            stream);
    if (e != hipSuccess) return fail_joined(hip_fail(e, "grouped_mlp_bwd dprobs"));
  }
  if (sd != nullptr) {
    st = wait_for(sd->s, stream, sd->ev[1]);
    if (st == MX_OK) st = run_gemm(pw1, MX_GROUP_K, mx::EPI_F32, sd->s, "grouped_mlp_bwd wgrad1");
    if (st != MX_OK) return fail_joined(st);
  }
  stage_mark(3, stream);
  if (sd == nullptr) {
    st = run_gemm(pw2, MX_GROUP_K, mx::EPI_F32, stream, "grouped_mlp_bwd wgrad2");
    if (st != MX_OK) return st;
  }
  stage_mark(4, stream);
  {
    const int tail = L.dev ? 0 : plan_split_tail(pd1, 2 * F, reinterpret_cast<float*>(at(workspace, L.split1)),
                                                 L.split1_bytes);
    st = run_gemm(pd1, MX_GROUP_M, mx::EPI_BF16, stream, "grouped_mlp_bwd dgrad1");
    if (st != MX_OK) return fail_joined(st);
    hipError_t e = mx::launch_split_reduce(mx::EPI_BF16, pd1.args, tail, stream);
    if (e != hipSuccess) return fail_joined(hip_fail(e, "grouped_mlp_bwd dgrad1 split reduce"));
  }
  stage_mark(5, stream);
  if (sd != nullptr) return wait_for(stream, sd->s, sd->ev[2]);
  st = run_gemm(pw1, MX_GROUP_K, mx::EPI_F32, stream, "grouped_mlp_bwd wgrad1");
  if (st != MX_OK) return st;
  stage_mark(6, stream);
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status grouped_mlp_bwd(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* dy, const float* probs,
                          const void* saved, size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                          int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = bwd_checks(L, dy, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  return bwd_impl(L, dy, probs, saved, nullptr, dx, dprobs, dw1, dw2, accumulate_wgrad, workspace,
                  reinterpret_cast<hipStream_t>(stream));
}

mx_status grouped_mlp_bwd_gather(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* dy_tokens,
                                 int64_t tokens, const int32_t* row_token, const float* probs, const void* saved,
                                 size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                                 int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd_gather";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = bwd_checks(L, dy_tokens, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  if (L.R > 0 && !row_token) return fail(MX_EINVAL, "%s: row_token is null", who);
  if (tokens < 0 || tokens > kI32Max) return fail(MX_ESHAPE, "%s: bad token count %lld", who, (long long)tokens);
  if (!aligned(row_token, 4)) return fail(MX_EALIGN, "%s: row_token must be 4-byte aligned", who);
  return bwd_impl(L, dy_tokens, probs, saved, nullptr, dx, dprobs, dw1, dw2, accumulate_wgrad, workspace,
                  reinterpret_cast<hipStream_t>(stream), row_token, tokens);
}

mx_status grouped_mlp_bwd_cached(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* dy,
                                 const float* probs, const void* cache, size_t cache_bytes, const void* saved,
                                 size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                                 int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd_cached";
  MlpLayout L;
  mx_status st = mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = bwd_checks(L, dy, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  WeightCacheLayout W;
  st = cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  const WeightCopies wc = weight_cache_copies(W, const_cast<void*>(cache));
  return bwd_impl(L, dy, probs, saved, &wc, dx, dprobs, dw1, dw2, accumulate_wgrad, workspace,
                  reinterpret_cast<hipStream_t>(stream));
}

mx_status grouped_mlp_sizes_device_split(const mx_mlp_dims* dims, size_t* fwd_workspace, size_t* saved,
                                         size_t* bwd_workspace) {
  g_err[0] = 0;
  MlpLayout L;
  mx_status st = mlp_layout(dims, nullptr, &L, "grouped_mlp_sizes_device_split", true);
  if (st != MX_OK) return st;
  if (fwd_workspace) *fwd_workspace = L.fwd_total;
  if (saved) *saved = L.saved_total;
  if (bwd_workspace) *bwd_workspace = L.bwd_total;
  return MX_OK;
}

mx_status grouped_mlp_fwd_device_split(const mx_mlp_dims* dims, const int64_t* split_sizes_dev, const void* x,
                                       int64_t tokens, const int32_t* row_token, const float* probs,
                                       const void* w1, const void* w2, const void* cache, size_t cache_bytes,
                                       void* y, void* saved, size_t saved_bytes, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd_device_split";
  MlpLayout L;
  mx_status st = mlp_layout(dims, nullptr, &L, who, true);
  if (st != MX_OK) return st;
  if (!split_sizes_dev) return fail(MX_EINVAL, "%s: split_sizes is null", who);
  if (!aligned(split_sizes_dev, 8)) return fail(MX_EALIGN, "%s: split_sizes must be 8-byte aligned", who);
  L.counts_dev = split_sizes_dev;
  st = fwd_checks(L, x, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  if (row_token) {
    if (tokens < 0 || tokens > kI32Max) return fail(MX_ESHAPE, "%s: bad token count %lld", who, (long long)tokens);
    if (!aligned(row_token, 4)) return fail(MX_EALIGN, "%s: row_token must be 4-byte aligned", who);
  }
  WeightCopies wc{};
  if (cache) {
    WeightCacheLayout W;
    st = cache_checks(L, cache, cache_bytes, &W, who);
    if (st != MX_OK) return st;
    wc = weight_cache_copies(W, const_cast<void*>(cache));
  } else {
    if (!w1 || !w2) return fail(MX_EINVAL, "%s: null pointer argument (w1, w2 or a weight cache)", who);
    if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte aligned", who);
  }
  return fwd_impl(L, x, probs, w1, w2, cache ? &wc : nullptr, y, saved, workspace,
                  reinterpret_cast<hipStream_t>(stream), row_token, row_token ? tokens : 0);
}

mx_status grouped_mlp_bwd_device_split(const mx_mlp_dims* dims, const int64_t* split_sizes_dev, const void* dy,
                                       int64_t tokens, const int32_t* row_token, const float* probs,
                                       const void* cache, size_t cache_bytes, const void* saved,
                                       size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                                       int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd_device_split";
  MlpLayout L;
  mx_status st = mlp_layout(dims, nullptr, &L, who, true);
  if (st != MX_OK) return st;
  if (!split_sizes_dev) return fail(MX_EINVAL, "%s: split_sizes is null", who);
  if (!aligned(split_sizes_dev, 8)) return fail(MX_EALIGN, "%s: split_sizes must be 8-byte aligned", who);
  L.counts_dev = split_sizes_dev;
  st = bwd_checks(L, dy, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  if (row_token) {
    if (tokens < 0 || tokens > kI32Max) return fail(MX_ESHAPE, "%s: bad token count %lld", who, (long long)tokens);
    if (!aligned(row_token, 4)) return fail(MX_EALIGN, "%s: row_token must be 4-byte aligned", who);
  }
  WeightCopies wc{};
  if (cache) {
    WeightCacheLayout W;
    st = cache_checks(L, cache, cache_bytes, &W, who);
    if (st != MX_OK) return st;
    wc = weight_cache_copies(W, const_cast<void*>(cache));
  }
  return bwd_impl(L, dy, probs, saved, cache ? &wc : nullptr, dx, dprobs, dw1, dw2, accumulate_wgrad, workspace,
                  reinterpret_cast<hipStream_t>(stream), row_token, row_token ? tokens : 0);
}

size_t mx_moe_dispatch_workspace_bytes(int64_t tokens, int32_t topk, int32_t num_experts) {
  if (tokens < 0 || topk < 1 || num_experts < 1 || num_experts > mx::kMaxGroups) return 0;
  const int64_t nblk = cdiv(tokens * topk, mx::kMoeBlock);
  return (size_t)((nblk * num_experts + 1) * 4);
}

}  // extern "C"

namespace {

// Token dispatch after the size checks; workspace null = the library's
// per-device scratch array (allocation-free variant).
mx_status moe_dispatch_impl(const char* who, const void* x, const int32_t* topk_idx, const float* topk_w,
                            int64_t tokens, int64_t hidden, int32_t topk, int32_t num_experts, void* x_perm,
                            float* probs_perm, int32_t* perm, int32_t* row_token, int64_t* counts, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (tokens < 0 || hidden <= 0 || hidden % 8) return fail(MX_ESHAPE, "%s: need tokens >= 0 and hidden a positive multiple of 8", who);
  if (topk < 1 || topk > 64) return fail(MX_EINVAL, "%s: topk %d outside [1, 64]", who, topk);
  if (num_experts < 1 || num_experts > mx::kMaxGroups)
    return fail(MX_EUNSUPPORTED, "%s: %d experts outside [1, %d]", who, num_experts, mx::kMaxGroups);
  if (tokens * topk > kI32Max || tokens * hidden > ((int64_t)1 << 40))
    return fail(MX_EUNSUPPORTED, "%s: too many routed rows", who);
  const bool own_scratch = workspace == nullptr && workspace_bytes == SIZE_MAX;
  if (!counts || (!workspace && !own_scratch) || (tokens > 0 && (!topk_idx || !perm || !row_token)))
    return fail(MX_EINVAL, "%s: null pointer argument", who);
  if ((x == nullptr) != (x_perm == nullptr))
    return fail(MX_EINVAL, "%s: x and x_perm must both be given or both be null (routing only)", who);
  if ((topk_w == nullptr) != (probs_perm == nullptr))
    return fail(MX_EINVAL, "%s: topk_w and probs_perm must both be given or both be null", who);
  if (!aligned(x, 16) || !aligned(x_perm, 16) || !aligned(topk_idx, 4) || !aligned(perm, 4) ||
      !aligned(row_token, 4) || !aligned(counts, 8) || !aligned(workspace, 4) || (topk_w && !aligned(topk_w, 4)) ||
      (probs_perm && !aligned(probs_perm, 4)))
    return fail(MX_EALIGN, "%s: x and x_perm must be 16-byte aligned, the index arrays 4-byte", who);
  const size_t need = mx_moe_dispatch_workspace_bytes(tokens, topk, num_experts);
  if (own_scratch) {
    if (need > (size_t)mx::kDispatchScratchWords * 4)
      return fail(MX_EUNSUPPORTED, "%s: %lld tokens x top-%d over %d experts need %zu bytes of scratch, above the "
                  "allocation-free limit of %lld bytes (ceil(tokens*topk/256)*experts + 1 <= %lld)", who,
                  (long long)tokens, topk, num_experts, need, (long long)mx::kDispatchScratchWords * 4,
                  (long long)mx::kDispatchScratchWords);
    int32_t* p = nullptr;
    hipError_t e = mx::dispatch_scratch(&p);
    if (e != hipSuccess) return hip_fail(e, "dispatch scratch address");
    workspace = p;
  } else if (workspace_bytes < need) {
    return fail(MX_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, need);
  }
  mx::MoeDispatchArgs a;
  a.x = x; a.topk_idx = topk_idx; a.topk_w = topk_w;
  a.tokens = tokens; a.hidden = hidden; a.topk = topk; a.experts = num_experts;
  a.x_perm = x_perm; a.probs_perm = probs_perm; a.perm = perm; a.row_token = row_token; a.counts = counts;
  a.workspace = reinterpret_cast<int32_t*>(workspace);
  hipError_t e = mx::launch_moe_dispatch(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_moe_dispatch launch");
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_moe_dispatch(const void* x, const int32_t* topk_idx, const float* topk_w, int64_t tokens,
                          int64_t hidden, int32_t topk, int32_t num_experts, void* x_perm, float* probs_perm,
                          int32_t* perm, int32_t* row_token, int64_t* counts, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  if (workspace == nullptr) return fail(MX_EINVAL, "mx_moe_dispatch: null pointer argument");
  return moe_dispatch_impl("mx_moe_dispatch", x, topk_idx, topk_w, tokens, hidden, topk, num_experts, x_perm,
                           probs_perm, perm, row_token, counts, workspace, workspace_bytes, stream);
}

mx_status mx_moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, const float* topk_w, int64_t tokens,
                                  int64_t hidden, int32_t topk, int32_t num_experts, void* x_perm,
                                  float* probs_perm, int32_t* perm, int32_t* row_token, int64_t* counts,
                                  void* stream) {
  g_err[0] = 0;
  return moe_dispatch_impl("mx_moe_dispatch_noalloc", x, topk_idx, topk_w, tokens, hidden, topk, num_experts,
                           x_perm, probs_perm, perm, row_token, counts, nullptr, SIZE_MAX, stream);
}

mx_status mx_moe_combine(const void* y_perm, const int32_t* perm, int64_t tokens, int64_t hidden, int32_t topk,
                         void* y, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_moe_combine";
  if (tokens < 0 || hidden <= 0 || hidden % 8) return fail(MX_ESHAPE, "%s: need tokens >= 0 and hidden a positive multiple of 8", who);
  if (topk < 1 || topk > 64) return fail(MX_EINVAL, "%s: topk %d outside [1, 64]", who, topk);
  if (tokens * topk > kI32Max) return fail(MX_EUNSUPPORTED, "%s: too many routed rows", who);
  if (tokens > 0 && (!y_perm || !perm || !y)) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(y_perm, 16) || !aligned(y, 16) || !aligned(perm, 4))
    return fail(MX_EALIGN, "%s: y_perm and y must be 16-byte aligned, perm 4-byte", who);
  hipError_t e = mx::launch_moe_combine(y_perm, perm, tokens, hidden, topk, y, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_moe_combine launch");
  return MX_OK;
}

mx_status mx_quantize_fp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                          uint8_t* s_col, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_quantize_fp4";
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MX_ESHAPE, "%s: need rows >= 0 and cols a positive multiple of 32", who);
  if (q_col != nullptr && rows % 32) return fail(MX_ESHAPE, "%s: the columnwise copy needs rows % 32 == 0", who);
  if (rows * (cols / 32) > kI32Max * (int64_t)256) return fail(MX_EUNSUPPORTED, "%s: tensor too large", who);
  if ((q == nullptr) != (s == nullptr) || (q_col == nullptr) != (s_col == nullptr))
    return fail(MX_EINVAL, "%s: codes and scales of a layout must both be given or both be null", who);
  if (q == nullptr && q_col == nullptr) return fail(MX_EINVAL, "%s: no output requested", who);
  if (rows > 0 && !x) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(q_col, 16))
    return fail(MX_EALIGN, "%s: x, q and q_col must be 16-byte aligned", who);
  hipError_t e = mx::launch_quantize_fp4(x, rows, cols, q, s, q_col, s_col, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_quantize_fp4 launch");
  return MX_OK;
}

mx_status mx_gemm_fp4(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s, int64_t m, int64_t n,
                      int64_t k, void* c, mx_dtype c_dtype, void* stream) {
  g_err[0] = 0;
  if (m < 0) return fail(MX_ESHAPE, "mx_gemm_fp4: need m >= 0");
  return gemm_fp4_impl("mx_gemm_fp4", a, a_s, b, b_s, &m, 1, n, k, c, c_dtype, stream);
}

mx_status mx_grouped_gemm_fp4(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                              const int64_t* group_sizes, int32_t groups, int64_t n, int64_t k, void* c,
                              mx_dtype c_dtype, void* stream) {
  g_err[0] = 0;
  return gemm_fp4_impl("mx_grouped_gemm_fp4", a, a_s, b, b_s, group_sizes, groups, n, k, c, c_dtype, stream);
}

mx_status mx_quantize_fp4_colwise_grouped(const void* x, int64_t rows, int64_t cols, const int64_t* group_sizes,
                                          int32_t groups, uint8_t* q_col, uint8_t* s_col, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_quantize_fp4_colwise_grouped";
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MX_ESHAPE, "%s: need rows >= 0 and cols a positive multiple of 32", who);
  if (groups < 1 || groups > mx::kMaxGroups) return fail(MX_EINVAL, "%s: need 1 <= groups <= %d", who, mx::kMaxGroups);
  mx_status st = check_groups(group_sizes, groups, rows, who);
  if (st != MX_OK) return st;
  if (!q_col || !s_col || (rows > 0 && !x)) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(x, 16) || !aligned(q_col, 16)) return fail(MX_EALIGN, "%s: x and q_col must be 16-byte aligned", who);
  mx::Fp4ColGroups gr{};
  gr.n = groups;
  int64_t r0 = 0, p0 = 0, t0 = 0;
  for (int g = 0; g < groups; ++g) {
    gr.row0[g] = r0;
    gr.pcol0[g] = p0;
    gr.tile0[g] = (int32_t)t0;
    r0 += group_sizes[g];
    p0 += pad32(group_sizes[g]);
    t0 += cdiv(group_sizes[g], 128);
  }
  gr.row0[groups] = r0;
  gr.pcol0[groups] = p0;
  gr.tile0[groups] = (int32_t)t0;
  if (t0 * cdiv(cols, 64) > kI32Max || p0 * cols > ((int64_t)1 << 40))
    return fail(MX_EUNSUPPORTED, "%s: tensor too large", who);
  hipError_t e = mx::launch_quantize_fp4_grouped(x, false, rows, cols, gr, q_col, s_col, nullptr, nullptr,
                                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_quantize_fp4_colwise_grouped launch");
  return MX_OK;
}

mx_status mx_grouped_gemm_fp4_wgrad(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                    const int64_t* group_sizes, int32_t groups, int64_t m, int64_t n, float* c,
                                    int32_t accumulate, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_grouped_gemm_fp4_wgrad";
  if (groups < 1 || groups > mx::kMaxGroups) return fail(MX_EINVAL, "%s: need 1 <= groups <= %d", who, mx::kMaxGroups);
  if (!group_sizes) return fail(MX_EINVAL, "%s: null group sizes", who);
  if (m < 0 || n < 0) return fail(MX_ESHAPE, "%s: need m >= 0 and n >= 0", who);
  mx::Fp4KGroups kg{};
  kg.n = groups;
  int64_t k = 0;
  for (int g = 0; g < groups; ++g) {
    if (group_sizes[g] < 0) return fail(MX_ESHAPE, "%s: negative group size", who);
    kg.k0[g] = k;
    k += pad32(group_sizes[g]);
  }
  kg.k0[groups] = k;
  if (k > ((int64_t)1 << 24)) return fail(MX_EUNSUPPORTED, "%s: padded rows above 2^24", who);
  const int64_t tiles = (int64_t)groups * cdiv(m, mx::kFp4GemmTileM) * cdiv(n, mx::kFp4GemmTileN);
  if (tiles > kI32Max || (int64_t)groups * m * n > ((int64_t)1 << 40))
    return fail(MX_EUNSUPPORTED, "%s: output too large", who);
  if (m == 0 || n == 0) return MX_OK;
  if (!c || (k > 0 && (!a || !a_s || !b || !b_s))) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16))
    return fail(MX_EALIGN, "%s: a, b and c must be 16-byte aligned", who);
  hipError_t e = mx::launch_gemm_fp4_group_k(a, a_s, b, b_s, kg, m, n, c, accumulate ? 1 : 0,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return MX_OK;
}

}  // extern "C"

extern "C" {

mx_status mx_quantize_nvfp4(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* s, uint8_t* q_col,
                            uint8_t* s_col, float* amax, void* stream) {
  g_err[0] = 0;
  const char* who = "mx_quantize_nvfp4";
  if (rows < 0 || cols <= 0 || cols % 16)
    return fail(MX_ESHAPE, "%s: need rows >= 0 and cols a positive multiple of 16", who);
  if (q_col != nullptr && rows % 16) return fail(MX_ESHAPE, "%s: the columnwise copy needs rows % 16 == 0", who);
  if ((q == nullptr) != (s == nullptr) || (q_col == nullptr) != (s_col == nullptr))
    return fail(MX_EINVAL, "%s: codes and scales of a layout must both be given or both be null", who);
  if (q == nullptr && q_col == nullptr) return fail(MX_EINVAL, "%s: no output requested", who);
  if (!amax || (rows > 0 && !x)) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(q_col, 8) || !aligned(amax, 4))
    return fail(MX_EALIGN, "%s: x must be 16-byte, q and q_col 8-byte and amax 4-byte aligned", who);
  if (cdiv(rows, 128) * cdiv(cols, 64) > kI32Max) return fail(MX_EUNSUPPORTED, "%s: tensor too large", who);
  hipError_t e = mx::launch_quantize_nvfp4(x, rows, cols, q, s, q_col, s_col, amax,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mx_quantize_nvfp4 launch");
  return MX_OK;
}

mx_status mx_gemm_nvfp4(const uint8_t* a, const uint8_t* a_s, const float* a_amax, const uint8_t* b,
                        const uint8_t* b_s, const float* b_amax, int64_t m, int64_t n, int64_t k, void* c,
                        mx_dtype c_dtype, void* stream) {
  g_err[0] = 0;
  if (m < 0) return fail(MX_ESHAPE, "mx_gemm_nvfp4: need m >= 0");
  return gemm_4bit_impl("mx_gemm_nvfp4", true, a, a_s, a_amax, b, b_s, b_amax, &m, 1, n, k, c, c_dtype, stream);
}

mx_status mx_grouped_gemm_nvfp4(const uint8_t* a, const uint8_t* a_s, const float* a_amax, const uint8_t* b,
                                const uint8_t* b_s, const float* b_amax, const int64_t* group_sizes, int32_t groups,
                                int64_t n, int64_t k, void* c, mx_dtype c_dtype, void* stream) {
  g_err[0] = 0;
  return gemm_4bit_impl("mx_grouped_gemm_nvfp4", true, a, a_s, a_amax, b, b_s, b_amax, group_sizes, groups, n, k, c,
                        c_dtype, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ MXFP4 MLP
// GroupedLinear -> ScaledSwiGLU -> GroupedLinear with every GEMM on MXFP4
// copies (the MLP of an FP4 layer: "TransformerEngine-accelerated Llama 3
// training with native PyTorch training loop", Layer-Wise Precision; the
// mxfp4 runs of "examples/llama: default-on fusion & DP-comm perf toggles").
// The steps are the MXFP8 MLP's; GEMM1 and dgrad2 leave fp32 results that
// the SwiGLU kernels turn into the requantized A / dH1.
namespace {

struct Fp4MlpLayout {
  int64_t E = 0, R = 0, H = 0, F = 0, P = 0;
  std::vector<int64_t> split;
  mx::Fp4ColGroups cg{};   // per-expert row tiles of the columnwise casts
  mx::Fp4KGroups kg{};     // per-expert padded k ranges of the weight gradients
  // forward workspace: rowwise X, W1, W2, H1 (fp32), rowwise A, GEMM2's
  // split-K partials
  size_t xq, xs, w1q, w1s, w2q, w2s, h1f, aq, as, split2, fwd_total;
  // saved: H1 (bf16), columnwise A, X, and per-expert columnwise W1, W2
  size_t h1, acq, acs, xcq, xcs, w1cq, w1cs, w2cq, w2cs, saved_total;
  // backward workspace: dY both layouts, dA (fp32), dH1 both layouts,
  // dprobs partials [F / 64, R], dgrad1's split-K partials
  size_t dyq, dys, dycq, dycs, da32, dhq, dhs, dhcq, dhcs, dpart, split1, bwd_total;
  size_t split_bytes;        // each of split2 / split1
};

mx_status fp4_mlp_layout(const mx_mlp_dims* d, const int64_t* split, Fp4MlpLayout* L, const char* who) {
  MlpLayout M;   // the MXFP8 MLP's checks of dims and split (shapes, limits, sums)
  mx_status st = mlp_layout(d, split, &M, who);
  if (st != MX_OK) return st;
  L->E = M.E;
  L->R = M.R;
  L->H = M.H;
  L->F = M.F;
  L->split = M.split;
  const int64_t E = L->E, R = L->R, H = L->H, F = L->F;
  L->cg.n = (int32_t)E;
  L->kg.n = (int32_t)E;
  int64_t r0 = 0, p0 = 0, t0 = 0;
  for (int g = 0; g < E; ++g) {
    L->cg.row0[g] = r0;
    L->cg.pcol0[g] = p0;
    L->cg.tile0[g] = (int32_t)t0;
    L->kg.k0[g] = p0;
    r0 += L->split[g];
    p0 += pad32(L->split[g]);
    t0 += cdiv(L->split[g], 128);
  }
  L->cg.row0[E] = r0;
  L->cg.pcol0[E] = p0;
  L->cg.tile0[E] = (int32_t)t0;
  L->kg.k0[E] = p0;
  L->P = p0;
  if (p0 > ((int64_t)1 << 24)) return fail(MX_EUNSUPPORTED, "%s: padded rows above 2^24", who);
  // launch grids: columnwise-cast tiles (widest input 2F), SwiGLU blocks, GEMM tiles
  const int64_t cast_tiles = t0 * cdiv(2 * L->F, 64), swiglu_blocks = cdiv(L->R * (L->F / 32), 256);
  const int64_t gemm_tiles = (cdiv(L->R, mx::kFp4GemmTileM) + L->E) * cdiv(2 * L->F, mx::kFp4GemmTileN);
  if (cast_tiles > kI32Max || swiglu_blocks > kI32Max || gemm_tiles > kI32Max)
    return fail(MX_EUNSUPPORTED, "%s: launch grid above 2^31", who);
  const int64_t P = L->P;
  size_t c = 0;
  L->xq = take(c, R * H / 2);
  L->xs = take(c, R * H / 32);
  L->w1q = take(c, E * 2 * F * H / 2);
  L->w1s = take(c, E * 2 * F * H / 32);
  L->w2q = take(c, E * H * F / 2);
  L->w2s = take(c, E * H * F / 32);
  L->h1f = take(c, R * 2 * F * 4);
  L->aq = take(c, R * F / 2);
  L->as = take(c, R * F / 32);
  // GEMM2 and dgrad1 (n = H): sum over experts of ceil(m_e/256) x ceil(H/256) tiles
  int64_t m_tiles = 0;
  for (int g = 0; g < E; ++g) m_tiles += cdiv(L->split[g], mx::kFp4GemmTileM);
  L->split_bytes = split_ws_bytes(m_tiles * cdiv(H, mx::kFp4GemmTileN));
  L->split2 = take(c, L->split_bytes);
  L->fwd_total = c;
  c = 0;
  L->h1 = take(c, R * 2 * F * 2);
  L->acq = take(c, F * P / 2);
  L->acs = take(c, F * P / 32);
  L->xcq = take(c, H * P / 2);
  L->xcs = take(c, H * P / 32);
  L->w1cq = take(c, E * H * 2 * F / 2);
  L->w1cs = take(c, E * H * 2 * F / 32);
  L->w2cq = take(c, E * F * H / 2);
  L->w2cs = take(c, E * F * H / 32);
  L->saved_total = c;
  c = 0;
  L->dyq = take(c, R * H / 2);
  L->dys = take(c, R * H / 32);
  L->dycq = take(c, H * P / 2);
  L->dycs = take(c, H * P / 32);
  L->da32 = take(c, R * F * 4);
  L->dhq = take(c, R * 2 * F / 2);
  L->dhs = take(c, R * 2 * F / 32);
  L->dhcq = take(c, 2 * F * P / 2);
  L->dhcs = take(c, 2 * F * P / 32);
  L->dpart = take(c, F / 64 * R * 4);
  L->split1 = take(c, L->split_bytes);
  L->bwd_total = c;
  return MX_OK;
}

mx_status fp4_step(hipError_t e, const char* what) { return e == hipSuccess ? MX_OK : hip_fail(e, what); }

// MXFP4 weight copies: rowwise W1 [E*2F, H] and W2 [E*H, F] for the forward
// GEMMs, and each expert's columnwise W1 [H, 2F] and W2 [F, H] for the dgrad
// GEMMs (codes two per byte, one scale byte per 32 values).
struct Fp4WeightCopies {
  const uint8_t *w1q, *w1s, *w2q, *w2s;
  const uint8_t *w1cq, *w1cs, *w2cq, *w2cs;
};

// Layout of an MXFP4 weight cache (grouped_mlp_fp4_quantize_weights): the
// four copies back to back, 256-byte aligned regions; offsets depend on E, H,
// F only.
struct Fp4WeightCacheLayout {
  size_t w1q, w1s, w2q, w2s, w1cq, w1cs, w2cq, w2cs, total;
};

Fp4WeightCacheLayout fp4_weight_cache_layout(int64_t E, int64_t H, int64_t F) {
  Fp4WeightCacheLayout W;
  size_t c = 0;
  W.w1q = take(c, E * 2 * F * H / 2); W.w1s = take(c, E * 2 * F * H / 32);
  W.w2q = take(c, E * H * F / 2); W.w2s = take(c, E * H * F / 32);
  W.w1cq = take(c, E * H * 2 * F / 2); W.w1cs = take(c, E * H * 2 * F / 32);
  W.w2cq = take(c, E * F * H / 2); W.w2cs = take(c, E * F * H / 32);
  W.total = c;
  return W;
}

Fp4WeightCopies fp4_weight_cache_copies(const Fp4WeightCacheLayout& W, const void* base) {
  return {at(base, W.w1q), at(base, W.w1s), at(base, W.w2q), at(base, W.w2s),
          at(base, W.w1cq), at(base, W.w1cs), at(base, W.w2cq), at(base, W.w2cs)};
}

// Both MXFP4 layouts of the bf16 master weights, one pass per expert and
// weight: rowwise into (w1q, w1s, w2q, w2s), columnwise into (w1cq, ...).
mx_status fp4_quantize_weights_into(int64_t E, int64_t H, int64_t F, const void* w1, const void* w2, uint8_t* w1q,
                                    uint8_t* w1s, uint8_t* w2q, uint8_t* w2s, uint8_t* w1cq, uint8_t* w1cs,
                                    uint8_t* w2cq, uint8_t* w2cs, hipStream_t stream, const char* who) {
  const uint8_t* w1b = static_cast<const uint8_t*>(w1);
  const uint8_t* w2b = static_cast<const uint8_t*>(w2);
  for (int64_t e = 0; e < E; ++e) {
    mx_status st = fp4_step(mx::launch_quantize_fp4(w1b + e * 2 * F * H * 2, 2 * F, H, w1q + e * 2 * F * H / 2,
                                                    w1s + e * 2 * F * H / 32, w1cq + e * H * 2 * F / 2,
                                                    w1cs + e * H * 2 * F / 32, stream), who);
    if (st != MX_OK) return st;
    st = fp4_step(mx::launch_quantize_fp4(w2b + e * H * F * 2, H, F, w2q + e * H * F / 2, w2s + e * H * F / 32,
                                          w2cq + e * F * H / 2, w2cs + e * F * H / 32, stream), who);
    if (st != MX_OK) return st;
  }
  return MX_OK;
}

mx_status fp4_cache_checks(const Fp4MlpLayout& L, const void* cache, size_t cache_bytes, Fp4WeightCacheLayout* W,
                           const char* who) {
  *W = fp4_weight_cache_layout(L.E, L.H, L.F);
  if (!cache) return fail(MX_EINVAL, "%s: weight cache is null", who);
  if (!aligned(cache, 256)) return fail(MX_EALIGN, "%s: weight cache must be 256-byte aligned", who);
  if (cache_bytes < W->total)
    return fail(MX_EWORKSPACE, "%s: weight cache %zu bytes < required %zu", who, cache_bytes, W->total);
  return MX_OK;
}

mx_status fwd_fp4_impl(const Fp4MlpLayout& L, const void* x, const float* probs, const void* w1, const void* w2,
                       const Fp4WeightCopies* wc, void* y, void* saved, void* workspace, hipStream_t stream,
                       const char* who) {
  uint8_t* W = static_cast<uint8_t*>(workspace);
  uint8_t* S = static_cast<uint8_t*>(saved);
  const bool train = saved != nullptr;
  const int64_t E = L.E, R = L.R, H = L.H, F = L.F;
  mx_status st;
  // X: rowwise (and, for the backward, the per-expert columnwise copy in the same pass)
  if (train)
    st = fp4_step(mx::launch_quantize_fp4_grouped(x, false, R, H, L.cg, S + L.xcq, S + L.xcs, W + L.xq, W + L.xs,
                                                  stream), who);
  else
    st = fp4_step(mx::launch_quantize_fp4(x, R, H, W + L.xq, W + L.xs, nullptr, nullptr, stream), who);
  if (st != MX_OK) return st;
  // weights: rowwise along H (W1) and F (W2); in training also each expert's
  // columnwise copy, [H, 2F] and [F, H], from the same pass. A weight cache
  // holds all of them already.
  const uint8_t *w1q = W + L.w1q, *w1s = W + L.w1s, *w2q = W + L.w2q, *w2s = W + L.w2s;
  if (wc) {
    w1q = wc->w1q; w1s = wc->w1s; w2q = wc->w2q; w2s = wc->w2s;
  } else if (train) {
    st = fp4_quantize_weights_into(E, H, F, w1, w2, W + L.w1q, W + L.w1s, W + L.w2q, W + L.w2s, S + L.w1cq,
                                   S + L.w1cs, S + L.w2cq, S + L.w2cs, stream, who);
    if (st != MX_OK) return st;
  } else {
    st = fp4_step(mx::launch_quantize_fp4(w1, E * 2 * F, H, W + L.w1q, W + L.w1s, nullptr, nullptr, stream), who);
    if (st != MX_OK) return st;
    st = fp4_step(mx::launch_quantize_fp4(w2, E * H, F, W + L.w2q, W + L.w2s, nullptr, nullptr, stream), who);
    if (st != MX_OK) return st;
  }
  // GEMM1 -> H1 (fp32)
  st = gemm_fp4_impl(who, W + L.xq, W + L.xs, w1q, w1s, L.split.data(), (int32_t)E, 2 * F, H, W + L.h1f, MX_F32,
                     stream);
  if (st != MX_OK) return st;
  // ScaledSwiGLU: A rowwise MXFP4; in training also H1 (bf16, saved) and A's
  // per-expert columnwise copy, from one pass over H1
  if (train) {
    mx::Fp4SwigluArgs sw{};
    sw.h1f = reinterpret_cast<const float*>(W + L.h1f);
    sw.h1_out = reinterpret_cast<uint16_t*>(S + L.h1);
    sw.probs = probs;
    sw.R = R;
    sw.F = F;
    st = fp4_step(mx::launch_swiglu_fp4_cast(false, sw, L.cg, S + L.acq, S + L.acs, W + L.aq, W + L.as, stream), who);
  } else {
    st = fp4_step(mx::launch_swiglu_fwd_fp4(reinterpret_cast<const float*>(W + L.h1f), probs, R, F, W + L.aq, W + L.as,
                                            stream), who);
  }
  if (st != MX_OK) return st;
  // GEMM2 -> Y (bf16)
  return gemm_fp4_impl(who, W + L.aq, W + L.as, w2q, w2s, L.split.data(), (int32_t)E, H, F, y, MX_BF16, stream,
                       reinterpret_cast<float*>(W + L.split2), L.split_bytes);
}

mx_status bwd_fp4_impl(const Fp4MlpLayout& L, const void* dy, const float* probs, const void* saved,
                       const Fp4WeightCopies* wc, void* dx, float* dprobs, float* dw1, float* dw2, int32_t accumulate,
                       void* workspace, hipStream_t stream, const char* who) {
  uint8_t* W = static_cast<uint8_t*>(workspace);
  const uint8_t* S = static_cast<const uint8_t*>(saved);
  const int64_t E = L.E, R = L.R, H = L.H, F = L.F;
  // columnwise weight copies: from saved (the forward cast them) or the cache
  const uint8_t* w1cq = wc ? wc->w1cq : S + L.w1cq;
  const uint8_t* w1cs = wc ? wc->w1cs : S + L.w1cs;
  const uint8_t* w2cq = wc ? wc->w2cq : S + L.w2cq;
  const uint8_t* w2cs = wc ? wc->w2cs : S + L.w2cs;
  // dY: rowwise (dgrad2) and per-expert columnwise (wgrad2) in one pass
  mx_status st = fp4_step(mx::launch_quantize_fp4_grouped(dy, false, R, H, L.cg, W + L.dycq, W + L.dycs, W + L.dyq,
                                                          W + L.dys, stream), who);
  if (st != MX_OK) return st;
  // dgrad2: dA = dY . W2 (fp32) on the columnwise W2 copies [F, H]
  st = gemm_fp4_impl(who, W + L.dyq, W + L.dys, w2cq, w2cs, L.split.data(), (int32_t)E, F, H, W + L.da32, MX_F32,
                     stream);
  if (st != MX_OK) return st;
  // SwiGLU backward: dH1 in both MXFP4 layouts from one pass over dA and the
  // saved H1, and dprobs from per-tile partial sums
  mx::Fp4SwigluArgs sw{};
  sw.da = reinterpret_cast<const float*>(W + L.da32);
  sw.h1 = reinterpret_cast<const uint16_t*>(S + L.h1);
  sw.dprobs_part = dprobs ? reinterpret_cast<float*>(W + L.dpart) : nullptr;
  sw.probs = probs;
  sw.R = R;
  sw.F = F;
  st = fp4_step(mx::launch_swiglu_fp4_cast(true, sw, L.cg, W + L.dhcq, W + L.dhcs, W + L.dhq, W + L.dhs, stream), who);
  if (st != MX_OK) return st;
  if (dprobs) {
    st = fp4_step(mx::launch_dprobs_reduce(reinterpret_cast<const float*>(W + L.dpart), dprobs, (int32_t)R,
                                           (int32_t)(F / 64), nullptr, stream), who);
    if (st != MX_OK) return st;
  }
  // dgrad1: dX = dH1 . W1 (bf16) on the columnwise W1 copies [H, 2F]
  st = gemm_fp4_impl(who, W + L.dhq, W + L.dhs, w1cq, w1cs, L.split.data(), (int32_t)E, H, 2 * F, dx, MX_BF16,
                     stream, reinterpret_cast<float*>(W + L.split1), L.split_bytes);
  if (st != MX_OK) return st;
  // weight gradients (fp32, stored or accumulated): dW2_e = dY_e^T A_e, dW1_e = dH1_e^T X_e
  st = fp4_step(mx::launch_gemm_fp4_group_k(W + L.dycq, W + L.dycs, S + L.acq, S + L.acs, L.kg, H, F, dw2, accumulate,
                                            stream), who);
  if (st != MX_OK) return st;
  return fp4_step(mx::launch_gemm_fp4_group_k(W + L.dhcq, W + L.dhcs, S + L.xcq, S + L.xcs, L.kg, 2 * F, H, dw1,
                                              accumulate, stream), who);
}

mx_status fp4_fwd_checks(const Fp4MlpLayout& L, const void* x, const float* probs, const void* y, const void* saved,
                         size_t saved_bytes, const void* workspace, size_t workspace_bytes, const char* who) {
  if (!x || !y || !workspace) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256) || (saved && !aligned(saved, 256)) ||
      (probs && !aligned(probs, 4)))
    return fail(MX_EALIGN, "%s: x, y must be 16-byte and workspace/saved 256-byte aligned", who);
  if (workspace_bytes < L.fwd_total)
    return fail(MX_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, L.fwd_total);
  if (saved && saved_bytes < L.saved_total)
    return fail(MX_EWORKSPACE, "%s: saved buffer %zu bytes < required %zu", who, saved_bytes, L.saved_total);
  return MX_OK;
}

mx_status fp4_bwd_checks(const Fp4MlpLayout& L, const void* dy, const float* probs, const void* saved,
                         size_t saved_bytes, const void* dx, const float* dprobs, const float* dw1, const float* dw2,
                         const void* workspace, size_t workspace_bytes, const char* who) {
  if (!dy || !saved || !dx || !dw1 || !dw2 || !workspace) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw1, 16) || !aligned(dw2, 16) || !aligned(saved, 256) ||
      !aligned(workspace, 256) || (probs && !aligned(probs, 4)) || (dprobs && !aligned(dprobs, 4)))
    return fail(MX_EALIGN, "%s: dy, dx, dw1, dw2 must be 16-byte and saved/workspace 256-byte aligned", who);
  if (saved_bytes < L.saved_total)
    return fail(MX_EWORKSPACE, "%s: saved buffer %zu bytes < required %zu", who, saved_bytes, L.saved_total);
  if (workspace_bytes < L.bwd_total)
    return fail(MX_EWORKSPACE, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, L.bwd_total);
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status grouped_mlp_fp4_sizes(const mx_mlp_dims* dims, const int64_t* split_sizes, size_t* fwd_workspace,
                                size_t* saved, size_t* bwd_workspace) {
  g_err[0] = 0;
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(dims, split_sizes, &L, "grouped_mlp_fp4_sizes");
  if (st != MX_OK) return st;
  if (fwd_workspace) *fwd_workspace = L.fwd_total;
  if (saved) *saved = L.saved_total;
  if (bwd_workspace) *bwd_workspace = L.bwd_total;
  return MX_OK;
}

mx_status grouped_mlp_fwd_fp4(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* x, const float* probs,
                              const void* w1, const void* w2, void* y, void* saved, size_t saved_bytes,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd_fp4";
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  if (!w1 || !w2) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte aligned", who);
  st = fp4_fwd_checks(L, x, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  return fwd_fp4_impl(L, x, probs, w1, w2, nullptr, y, saved, workspace, reinterpret_cast<hipStream_t>(stream), who);
}

mx_status grouped_mlp_bwd_fp4(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* dy, const float* probs,
                              const void* saved, size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                              int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd_fp4";
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fp4_bwd_checks(L, dy, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  return bwd_fp4_impl(L, dy, probs, saved, nullptr, dx, dprobs, dw1, dw2, accumulate_wgrad ? 1 : 0, workspace,
                      reinterpret_cast<hipStream_t>(stream), who);
}

mx_status grouped_mlp_fp4_weight_cache_bytes(const mx_mlp_dims* dims, size_t* bytes) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fp4_weight_cache_bytes";
  if (!bytes) return fail(MX_EINVAL, "%s: bytes is null", who);
  if (!dims) return fail(MX_EINVAL, "%s: dims is null", who);
  // the cache does not depend on the routed rows: check the rest with R = 0
  mx_mlp_dims d = *dims;
  d.rows = 0;
  std::vector<int64_t> zeros(d.num_experts > 0 && d.num_experts <= mx::kMaxGroups ? d.num_experts : 1, 0);
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(&d, zeros.data(), &L, who);
  if (st != MX_OK) return st;
  *bytes = fp4_weight_cache_layout(L.E, L.H, L.F).total;
  return MX_OK;
}

mx_status grouped_mlp_fp4_quantize_weights(const mx_mlp_dims* dims, const void* w1, const void* w2, void* cache,
                                           size_t cache_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fp4_quantize_weights";
  if (!dims) return fail(MX_EINVAL, "%s: dims is null", who);
  mx_mlp_dims d = *dims;
  d.rows = 0;
  std::vector<int64_t> zeros(d.num_experts > 0 && d.num_experts <= mx::kMaxGroups ? d.num_experts : 1, 0);
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(&d, zeros.data(), &L, who);
  if (st != MX_OK) return st;
  Fp4WeightCacheLayout W;
  st = fp4_cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  if (!w1 || !w2) return fail(MX_EINVAL, "%s: null pointer argument", who);
  if (!aligned(w1, 16) || !aligned(w2, 16)) return fail(MX_EALIGN, "%s: w1, w2 must be 16-byte aligned", who);
  uint8_t* c = static_cast<uint8_t*>(cache);
  return fp4_quantize_weights_into(L.E, L.H, L.F, w1, w2, c + W.w1q, c + W.w1s, c + W.w2q, c + W.w2s, c + W.w1cq,
                                   c + W.w1cs, c + W.w2cq, c + W.w2cs, reinterpret_cast<hipStream_t>(stream), who);
}

mx_status grouped_mlp_fwd_fp4_cached(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* x,
                                     const float* probs, const void* cache, size_t cache_bytes, void* y, void* saved,
                                     size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_fwd_fp4_cached";
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fp4_fwd_checks(L, x, probs, y, saved, saved_bytes, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  Fp4WeightCacheLayout W;
  st = fp4_cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  const Fp4WeightCopies wc = fp4_weight_cache_copies(W, cache);
  return fwd_fp4_impl(L, x, probs, nullptr, nullptr, &wc, y, saved, workspace, reinterpret_cast<hipStream_t>(stream),
                      who);
}

mx_status grouped_mlp_bwd_fp4_cached(const mx_mlp_dims* dims, const int64_t* split_sizes, const void* dy,
                                     const float* probs, const void* cache, size_t cache_bytes, const void* saved,
                                     size_t saved_bytes, void* dx, float* dprobs, float* dw1, float* dw2,
                                     int32_t accumulate_wgrad, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  const char* who = "grouped_mlp_bwd_fp4_cached";
  Fp4MlpLayout L;
  mx_status st = fp4_mlp_layout(dims, split_sizes, &L, who);
  if (st != MX_OK) return st;
  st = fp4_bwd_checks(L, dy, probs, saved, saved_bytes, dx, dprobs, dw1, dw2, workspace, workspace_bytes, who);
  if (st != MX_OK) return st;
  Fp4WeightCacheLayout W;
  st = fp4_cache_checks(L, cache, cache_bytes, &W, who);
  if (st != MX_OK) return st;
  const Fp4WeightCopies wc = fp4_weight_cache_copies(W, cache);
  return bwd_fp4_impl(L, dy, probs, saved, &wc, dx, dprobs, dw1, dw2, accumulate_wgrad ? 1 : 0, workspace,
                      reinterpret_cast<hipStream_t>(stream), who);
}

}  // extern "C"
