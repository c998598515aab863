// After the LM head: merge the per-tile (max, argmax, 2nd max, sum exp)
// records of each drafted row, commit positions by confidence, and the
// greedy verification of a drafted block.
#include "kernels.h"

namespace dflash {

namespace {

__global__ __launch_bounds__(256) void lm_merge_kernel(int ntiles,
                                                       const Top2* part,
                                                       RowResult* res) {
  __shared__ Top2 wres[4];
  const int row = blockIdx.x;
  const Top2* src = part + (int64_t)row * ntiles;
  Top2 t = top2_empty();
  for (int k = threadIdx.x; k < ntiles; k += 256) t = top2_merge(t, src[k]);
  t = top2_wave(t);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wres[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    Top2 a = wres[0];
    a = top2_merge(a, wres[1]);
    a = top2_merge(a, wres[2]);
    a = top2_merge(a, wres[3]);
    RowResult rr;
    rr.token = a.i1;
    rr.conf = 1.f / a.s;  // exp(max - logsumexp)
    rr.margin = a.m1 - a.m2;
    rr.lse = a.m1 + logf(a.s);
    res[row] = rr;
  }
}

// One wave per sequence; lane i is block index i.  Masked lanes read their
// compact row (rank among masked positions by index), rank themselves by
// confidence (ties -> lower index) and commit if within the pass's quota.
__global__ __launch_bounds__(64) void commit_kernel(
    int K, int n_cap, int quota, int last, const RowResult* res, BlockState st,
    int32_t* draft, float* conf_out, float* margin_out) {
  const int b = blockIdx.x, i = threadIdx.x;
  const bool in = i < K;
  const bool masked = in && !st.committed[b * K + i];
  const unsigned long long ball = __ballot(masked);
  const unsigned long long below = (i == 0) ? 0ull : (ball & ((1ull << i) - 1ull));
  const int rank_idx = __popcll(below);
  RowResult rr{0, 0.f, 0.f, 0.f};
  if (masked) rr = res[b * n_cap + rank_idx];
  const float cf = masked ? rr.conf : -1.f;
  int better = 0;
  for (int j = 0; j < K; ++j) {
    const float cj = __shfl(cf, j, 64);
    const int mj = (int)((ball >> j) & 1ull);
    if (mj && (cj > cf || (cj == cf && j < i))) ++better;
  }
  if (masked && (last || better < quota)) {
    st.tokens[b * K + i] = rr.token;
    st.committed[b * K + i] = 1;
    const int64_t o = (int64_t)b * (K - 1) + (i - 1);
    draft[o] = rr.token;
    if (conf_out) conf_out[o] = rr.conf;
    if (margin_out) margin_out[o] = rr.margin;
  }
}

__global__ void verify_kernel(int B, int K, const int32_t* draft,
                              const int32_t* target, int32_t* accept,
                              int32_t* next_anchor) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* d = draft + (int64_t)b * (K - 1);
  const int32_t* t = target + (int64_t)b * K;
  int tau = 0;
  while (tau < K - 1 && d[tau] == t[tau]) ++tau;
  accept[b] = tau + 1;
  next_anchor[b] = t[tau];
}

}  // namespace

hipError_t launch_lm_merge(int rows, int ntiles, const Top2* part,
                           RowResult* res, hipStream_t s) {
  hipLaunchKernelGGL(lm_merge_kernel, dim3(rows), dim3(256), 0, s, ntiles,
                     part, res);
  return hipGetLastError();
}

hipError_t launch_commit(int B, int K, int n_cap, int commit, bool last,
                         const RowResult* res, BlockState st, int32_t* draft,
                         float* conf, float* margin, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(64), 0, s, K, n_cap, commit,
                     last ? 1 : 0, res, st, draft, conf, margin);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int K, const int32_t* draft,
                         const int32_t* target, int32_t* accept,
                         int32_t* next_anchor, hipStream_t s) {
  hipLaunchKernelGGL(verify_kernel, dim3((B + 63) / 64), dim3(64), 0, s, B, K,
                     draft, target, accept, next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
