// After the LM head: merge the per-tile (max, argmax, 2nd max, sum exp)
// records of each drafted row, commit positions by confidence, and the
// greedy verification of a drafted block.
#include "kernels.h"

namespace dflash {

namespace {

// Stage 1: each workgroup merges one contiguous chunk of a row's vocabulary
// tiles (tile order within the chunk is fixed by the thread mapping).
__global__ __launch_bounds__(256) void lm_merge_kernel(int ntiles,
                                                       const Top2* part,
                                                       Top2* part2) {
  __shared__ Top2 wres[4];
  const int row = blockIdx.x / kMergeChunks, ch = blockIdx.x % kMergeChunks;
  const int per = (ntiles + kMergeChunks - 1) / kMergeChunks;
  const int t0 = ch * per, t1 = min(ntiles, t0 + per);
  const Top2* src = part + (int64_t)row * ntiles;
  Top2 t = top2_empty();
  for (int k = t0 + threadIdx.x; k < t1; k += 256) t = top2_merge(t, src[k]);
  t = top2_wave(t);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wres[wave] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    Top2 a = wres[0];
    a = top2_merge(a, wres[1]);
    a = top2_merge(a, wres[2]);
    a = top2_merge(a, wres[3]);
    part2[(int64_t)row * kMergeChunks + ch] = a;
  }
}

// One wave per sequence; lane i is block index i.  A masked lane merges the
// chunk records of its LM-head row (rank among masked positions by index),
// then ranks itself by confidence (ties -> lower index) and commits if within
// the pass's quota.
__global__ __launch_bounds__(64) void commit_kernel(
    int K, int n_cap, int quota, int last, const Top2* part2, BlockState st,
    int32_t* draft, float* conf_out, float* margin_out) {
  const int b = blockIdx.x, i = threadIdx.x;
  const bool masked = i < K && !st.committed[b * K + i];
  const unsigned long long ball = __ballot(masked);
  const unsigned long long below = (i == 0) ? 0ull : (ball & ((1ull << i) - 1ull));
  const int rank_idx = __popcll(below);
  Top2 r = top2_empty();
  if (masked) {
    const Top2* src = part2 + (int64_t)(b * n_cap + rank_idx) * kMergeChunks;
    Top2 c[kMergeChunks];
#pragma unroll
    for (int k = 0; k < kMergeChunks; ++k) c[k] = src[k];
#pragma unroll
    for (int k = 0; k < kMergeChunks; ++k) r = top2_merge(r, c[k]);
  }
  const float cf = masked ? 1.f / r.s : -1.f;  // exp(max - logsumexp)
  int better = 0;
  for (int j = 0; j < K; ++j) {
    const float cj = __shfl(cf, j, 64);
    const int mj = (int)((ball >> j) & 1ull);
    if (mj && (cj > cf || (cj == cf && j < i))) ++better;
  }
  if (masked && (last || better < quota)) {
    st.tokens[b * K + i] = r.i1;
    st.committed[b * K + i] = 1;
    const int64_t o = (int64_t)b * (K - 1) + (i - 1);
    draft[o] = r.i1;
    if (conf_out) conf_out[o] = cf;
    if (margin_out) margin_out[o] = r.m1 - r.m2;
  }
}

// One thread per sequence: a mismatch bit per drafted position (loads are
// independent of each other), tau = index of the first set bit.
__global__ void verify_kernel(int B, int K, const int32_t* draft,
                              const int32_t* target, int32_t* accept,
                              int32_t* next_anchor) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t* d = draft + (int64_t)b * (K - 1);
  const int32_t* t = target + (int64_t)b * K;
  unsigned long long mism = 1ull << (K - 1);  // sentinel after the draft
#pragma unroll 16
  for (int j = 0; j < K - 1; ++j)
    if (d[j] != t[j]) mism |= 1ull << j;
  const int tau = __ffsll((long long)mism) - 1;
  accept[b] = tau + 1;
  next_anchor[b] = t[tau];
}

}  // namespace

hipError_t launch_lm_merge(int rows, int ntiles, const Top2* part, Top2* part2,
                           hipStream_t s) {
  hipLaunchKernelGGL(lm_merge_kernel, dim3(rows * kMergeChunks), dim3(256), 0,
                     s, ntiles, part, part2);
  return hipGetLastError();
}

hipError_t launch_commit(int B, int K, int n_cap, int commit, bool last,
                         const Top2* part2, BlockState st, int32_t* draft,
                         float* conf, float* margin, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(64), 0, s, K, n_cap, commit,
                     last ? 1 : 0, part2, st, draft, conf, margin);
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
