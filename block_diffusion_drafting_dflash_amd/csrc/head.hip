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

// One workgroup per sequence.  Wave w merges the records of the LM-head
// rows of block positions w, w + 16, ... (a masked position's row is its
// rank among the masked positions): nrec records per row, lane k taking
// records k, k + 64, ... in order (loaded four at a time), then a
// butterfly.  Wave 0 then ranks the
// masked positions by confidence (ties -> lower index) and commits those
// within the pass's quota.
constexpr int kCommitWaves = 16;

__global__ __launch_bounds__(64 * kCommitWaves) void commit_kernel(
    int K, int n_cap, int quota, int last, const Top2* part, int nrec,
    BlockState st, int32_t* draft, float* conf_out, float* margin_out) {
  __shared__ Top2 res[64];
  __shared__ unsigned long long ball_s;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const bool m = lane < K && !st.committed[b * K + lane];
    const unsigned long long ball = __ballot(m);
    if (lane == 0) ball_s = ball;
  }
  __syncthreads();
  const unsigned long long ball = ball_s;
  for (int i = wave; i < K; i += kCommitWaves) {
    if (!((ball >> i) & 1ull)) continue;  // uniform per wave
    const int rank_idx = __popcll(ball & ((1ull << i) - 1ull));
    const Top2* src = part + (int64_t)(b * n_cap + rank_idx) * nrec;
    // lane records issued in batches of kCommitBatch, merged in order
    constexpr int kCommitBatch = 4;
    Top2 r = top2_empty();
    for (int k0 = 0; k0 < nrec; k0 += 64 * kCommitBatch) {
      Top2 t[kCommitBatch];
#pragma unroll
      for (int u = 0; u < kCommitBatch; ++u) {
        const int k = k0 + u * 64 + lane;
        t[u] = k < nrec ? src[k] : top2_empty();
      }
#pragma unroll
      for (int u = 0; u < kCommitBatch; ++u) r = top2_merge(r, t[u]);
    }
    r = top2_wave(r);
    if (lane == 0) res[i] = r;
  }
  __syncthreads();
  if (wave != 0) return;
  const int i = lane;
  const bool masked = (ball >> i) & 1ull;
  const Top2 r = masked ? res[i] : top2_empty();
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
                         const Top2* part, int nrec, BlockState st,
                         int32_t* draft, float* conf, float* margin,
                         hipStream_t s) {
  if (K > 64 || nrec < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(64 * kCommitWaves), 0, s, K,
                     n_cap, commit, last ? 1 : 0, part, nrec, st, draft, conf,
                     margin);
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
