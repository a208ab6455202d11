// Token dispatch and combine around the grouped MLP: each token activates a
// few experts ("Efficient MoE training for biological foundation models",
// Dense vs. MoE scaling), and GroupedLinear takes the input tokens of each
// expert gathered into one group with per-expert counts, split_sizes (Key
// technical approaches, item 1).
//
// Dispatch: the (token, slot) entries of the top-k choices, in token order,
// become routed rows ordered by expert, then token. Four passes, all
// deterministic (no global atomics):
//   1. per block of 256 entries, a histogram of experts (LDS counters);
//   2. one workgroup turns the histograms into the first routed row of each
//      (block, expert) and writes the per-expert counts and the total;
//   3. each entry's routed row = its (block, expert) base + its rank among the
//      block's earlier entries of the same expert;
//   4. the token rows are copied to their routed rows, 16 bytes per lane
//      (skipped in routing-only mode, where the MLP's X cast gathers).
// Entries whose expert lies outside [0, E) are dropped (perm -1).
// Combine: y[t] = sum over slots of the routed output rows of token t, in
// fp32 in slot order, rounded once to bf16.
#include <mutex>

#include "mx_device.h"
#include "mx_internal.h"

namespace mx {

// Scratch of the allocation-free dispatch (mx_moe_dispatch_noalloc): the
// per-block expert histograms, then the per-(block, expert) first routed rows,
// and the routed-row total, kDispatchScratchWords int32 at most. Every word
// the dispatch reads is written earlier in the same call, so the array needs
// no clearing. One copy per GPU, held until the process ends; calls that
// overlap on one GPU share it and race.
static __device__ __align__(256) int32_t scratch[kDispatchScratchWords];

hipError_t dispatch_scratch(int32_t** out) {
  static std::mutex mu;
  static int32_t* ptr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    // the device address of this device's copy (the host-side name is only a
    // stand-in and must never reach a kernel)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void moe_hist_kernel(const int32_t* idx, int64_t n, int32_t E, int32_t* hist) {
  __shared__ int32_t h[kMaxGroups];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kMoeBlock + tid;
  if (i < n) {
    const int32_t e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One workgroup: hist[b][e] becomes the first routed row of expert e's
// entries in block b; counts[e] (int64) and the total (hist[nblk * E]).
__global__ __launch_bounds__(256) void moe_scan_kernel(int32_t* hist, int32_t nblk, int32_t E, int64_t* counts) {
  __shared__ int32_t tot[kMaxGroups];
  __shared__ int32_t off[kMaxGroups];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) {
    int32_t s = 0;
    for (int b = 0; b < nblk; ++b) {
      const int32_t c = hist[(int64_t)b * E + e];
      hist[(int64_t)b * E + e] = s;
      s += c;
    }
    tot[e] = s;
    counts[e] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t s = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = s;
      s += tot[e];
    }
    hist[(int64_t)nblk * E] = s;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    for (int b = 0; b < nblk; ++b) hist[(int64_t)b * E + e] += off[e];
}

__global__ __launch_bounds__(256) void moe_place_kernel(const int32_t* idx, const float* w, int64_t n, int32_t k,
                                                        int32_t E, const int32_t* base, int32_t* perm,
                                                        int32_t* row_token, float* probs_perm) {
  __shared__ int32_t ex[kMoeBlock];
  const int tid = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * kMoeBlock + tid;
  int32_t e = -1;
  if (i < n) {
    e = idx[i];
    if (e < 0 || e >= E) e = -1;
  }
  ex[tid] = e;
  __syncthreads();
  if (i >= n) return;
  if (e < 0) {
    perm[i] = -1;
    return;
  }
  int32_t rank = 0;
  for (int j = 0; j < tid; ++j) rank += ex[j] == e;
  const int32_t r = base[(int64_t)blockIdx.x * E + e] + rank;
  perm[i] = r;
  row_token[r] = (int32_t)(i / k);
  if (probs_perm != nullptr) probs_perm[r] = w[i];
}

// Workgroup r copies token row_token[r] into routed row r (rows past the
// total of valid entries are left alone).
__global__ __launch_bounds__(256) void moe_gather_kernel(const uint4* x, const int32_t* row_token, const int32_t* total,
                                                         int64_t row_vec, uint4* x_perm) {
  const int64_t r = blockIdx.x;
  if (r >= *total) return;
  const int64_t t = row_token[r];
  for (int64_t c = threadIdx.x; c < row_vec; c += 256) x_perm[r * row_vec + c] = x[t * row_vec + c];
}

__global__ __launch_bounds__(256) void moe_combine_kernel(const uint4* y_perm, const int32_t* perm, int32_t k,
                                                          int64_t row_vec, uint4* y) {
  const int64_t t = blockIdx.x;
  for (int64_t c = threadIdx.x; c < row_vec; c += 256) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int32_t r = perm[t * k + j];
      if (r < 0) continue;
      const uint4 v = y_perm[(int64_t)r * row_vec + c];
      a[0] += bf16_lo(v.x); a[1] += bf16_hi(v.x);
      a[2] += bf16_lo(v.y); a[3] += bf16_hi(v.y);
      a[4] += bf16_lo(v.z); a[5] += bf16_hi(v.z);
      a[6] += bf16_lo(v.w); a[7] += bf16_hi(v.w);
    }
    uint4 o;
    o.x = pack_bf16x2(a[0], a[1]);
    o.y = pack_bf16x2(a[2], a[3]);
    o.z = pack_bf16x2(a[4], a[5]);
    o.w = pack_bf16x2(a[6], a[7]);
    y[t * row_vec + c] = o;
  }
}

hipError_t launch_moe_dispatch(const MoeDispatchArgs& a, hipStream_t stream) {
  const int64_t n = a.tokens * a.topk;
  const int32_t nblk = (int32_t)((n + kMoeBlock - 1) / kMoeBlock);
  const int64_t row_vec = a.hidden * 2 / 16;
  if (nblk > 0)
    hipLaunchKernelGGL(moe_hist_kernel, dim3(nblk), dim3(256), 0, stream, a.topk_idx, n, a.experts, a.workspace);
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(256), 0, stream, a.workspace, nblk, a.experts, a.counts);
  if (nblk == 0) return hipGetLastError();
  hipLaunchKernelGGL(moe_place_kernel, dim3(nblk), dim3(256), 0, stream, a.topk_idx, a.topk_w, n, a.topk,
                     a.experts, a.workspace, a.perm, a.row_token, a.probs_perm);
  if (a.x_perm == nullptr) return hipGetLastError();     // routing only
  hipLaunchKernelGGL(moe_gather_kernel, dim3((unsigned)n), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(a.x), a.row_token, a.workspace + (int64_t)nblk * a.experts,
                     row_vec, reinterpret_cast<uint4*>(a.x_perm));
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* y_perm, const int32_t* perm, int64_t tokens, int64_t hidden, int32_t topk,
                              void* y, hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)tokens), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(y_perm), perm, topk, hidden * 2 / 16, reinterpret_cast<uint4*>(y));
  return hipGetLastError();
}

}  // namespace mx
