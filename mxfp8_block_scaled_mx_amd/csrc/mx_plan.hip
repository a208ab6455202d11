// Group tables of the fused MLP built on the device from per-expert row
// counts that live in device memory ("Efficient MoE training for biological
// foundation models", Key technical approaches item 1: GroupedLinear takes
// the per-expert token counts, split_sizes). Counts produced on the device,
// such as the token dispatch's, then feed the grouped GEMMs and the
// activation casts without a copy to the host and a wait for it.
//
// One workgroup: thread 0 forms the prefix sums (E <= 128), then one thread
// per expert writes its entries of every table. The kernels that read the
// tables launch worst-case grids sized on the host from R and E alone.
#include "mx_internal.h"

namespace mx {

__global__ __launch_bounds__(256) void mlp_dev_plan_kernel(MlpDevPlanArgs a) {
  __shared__ int32_t m[kMaxGroups];         // clamped rows of expert e
  __shared__ int32_t r0[kMaxGroups + 1];    // first routed row
  __shared__ int32_t p0[kMaxGroups + 1];    // first column of the columnwise layouts (32-row padded groups)
  __shared__ int32_t q0[kMaxGroups + 1];    // first 128-column step of the k-tiled columnwise scales
  __shared__ int32_t t128[kMaxGroups + 1];  // first 128-row tile (activation casts)
  __shared__ int32_t t256[kMaxGroups + 1];  // first 256-row tile (group-M GEMMs)
  __shared__ int32_t slot_m[kMaxGroups];    // group-M slot (non-empty experts in order)
  __shared__ int32_t slot_k[kMaxGroups];    // group-K slot (longest contraction first)
  __shared__ int32_t n_nonempty;
  const int t = threadIdx.x;
  const int E = a.E;
  if (t == 0) {
    int64_t run = 0;
    int32_t pp = 0, qq = 0, tq = 0, tm = 0, nz = 0;
    for (int e = 0; e < E; ++e) {
      int64_t c = a.counts[e];
      if (c < 0) c = 0;
      if (c > (int64_t)a.R - run) c = (int64_t)a.R - run;
      const int32_t ci = (int32_t)c;
      m[e] = ci;
      r0[e] = (int32_t)run;
      p0[e] = pp;
      q0[e] = qq;
      t128[e] = tq;
      t256[e] = tm;
      slot_m[e] = nz;
      run += c;
      pp += (ci + 31) / 32 * 32;
      qq += (ci + 127) / 128;
      tq += (ci + 127) / 128;
      tm += (ci + 255) / 256;
      nz += ci > 0 ? 1 : 0;
    }
    r0[E] = (int32_t)run;
    p0[E] = pp;
    q0[E] = qq;
    t128[E] = tq;
    t256[E] = tm;
    n_nonempty = nz;
  }
  __syncthreads();
  if (t < E) {
    int rank = 0;
    for (int e = 0; e < E; ++e) rank += (m[e] > m[t] || (m[e] == m[t] && e < t)) ? 1 : 0;
    slot_k[t] = rank;
  }
  __syncthreads();

  MlpDevPlan* P = a.plan;
  if (t <= E) {
    P->act.row0[t] = r0[t];
    P->act.pcol0[t] = p0[t];
    P->act.tile0[t] = t128[t];
    P->act.q0[t] = q0[t];
  }
  if (t == 0) {
    P->act.n = E;
    P->rows = r0[E];
    P->pad_ = 0;
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    GemmGroups& G = P->m[j];
    const int32_t tn = a.m_tiles_n[j];
    if (t < E && m[t] > 0) {
      const int s = slot_m[t];
      G.tile0[s] = t256[t] * tn;
      G.gid[s] = t;
      G.a0[s] = r0[t];
      G.len[s] = m[t];
      G.pc0[s] = p0[t];
      G.q0[s] = q0[t];
    }
    if (t == 0) {
      G.n = n_nonempty;
      G.interleave = 0;
      G.tile0[n_nonempty] = t256[E] * tn;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    GemmGroups& G = P->k[j];
    const int32_t per_slot = a.k_slot_tiles[j];
    if (t < E) {
      const int s = slot_k[t];
      G.tile0[s] = s * per_slot;
      G.gid[s] = t;
      G.a0[s] = p0[t];
      G.len[s] = (m[t] + 31) / 32 * 32;
      G.pc0[s] = p0[t];
      G.q0[s] = q0[t];
    }
    if (t == 0) {
      G.n = E;
      G.interleave = a.k_interleave[j];
      G.tile0[E] = E * per_slot;
    }
  }
}

hipError_t launch_mlp_dev_plan(const MlpDevPlanArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(mlp_dev_plan_kernel, dim3(1), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace mx
