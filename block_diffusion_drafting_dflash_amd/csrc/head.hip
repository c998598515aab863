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

// One workgroup per sequence.  Wave w merges the records of LM-head rows
// w, w + 16, ... of the sequence (row = rank of a still-masked position):
// nrec records per row, lane k taking records k, k + 64, ... in order
// (loaded four at a time), then a butterfly.  The rows are taken by rank, so
// the loads need no block state; ranks past the masked count hold records
// of zeroed rows and are never read back.  Wave 0 then maps each masked
// position to its rank, ranks the positions by confidence (ties -> lower
// index) and commits those within the pass's quota.
constexpr int kCommitWaves = 16;

__global__ __launch_bounds__(64 * kCommitWaves) void commit_kernel(
    int K, int n_cap, int quota, int last, const Top2* part, int nrec,
    BlockState st, int32_t* draft, float* conf_out, float* margin_out) {
  __shared__ Top2 res[64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int rk = wave; rk < n_cap; rk += kCommitWaves) {
    const Top2* src = part + (int64_t)(b * n_cap + rk) * nrec;
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
    if (lane == 0) res[rk] = r;
  }
  unsigned long long ball = 0;
  if (wave == 0) {
    const bool m = lane < K && !st.committed[b * K + lane];
    ball = __ballot(m);
  }
  __syncthreads();
  if (wave != 0) return;
  const int i = lane;
  const bool masked = (ball >> i) & 1ull;
  const int rank = __popcll(ball & ((1ull << i) - 1ull));
  const Top2 r = masked && rank < n_cap ? res[rank] : top2_empty();
  const float cf = masked ? 1.f / r.s : -1.f;  // exp(max - logsumexp)
  int better = 0;
  for (int j = 0; j < K; ++j) {
    const float cj = __shfl(cf, j, 64);
    const int mj = (int)((ball >> j) & 1ull);
    if (mj && (cj > cf || (cj == cf && j < i))) ++better;
  }
  if (masked && (last || better < quota)) {
    // a row whose maximum is not a finite logit (NaN activations leave the
    // record empty): id -1, flagged
    const bool ok = r.m1 > -INFINITY && r.m1 < INFINITY;
    if (!ok) set_error(st.err, DFLASH_DEVERR_TOKEN);
    const int tok = ok ? r.i1 : -1;
    st.tokens[b * K + i] = tok;
    st.committed[b * K + i] = 1;
    const int64_t o = (int64_t)b * (K - 1) + (i - 1);
    draft[o] = tok;
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

// Speculative-sampling verification, one workgroup of 16 waves per sequence.
// Wave 0 decides the acceptances.  The draw's weights are summed in
// 64-element tiles (coalesced loads, a fixed butterfly per tile), the tiles
// in index order within segments of 64 tiles, the segments in order; the draw
// walks segments, tiles and the tile's elements in that order and takes the
// first whose running sum exceeds u times the total (if rounding leaves the
// target at the very end, the last entry of positive weight).
constexpr int kSampWaves = 16;
constexpr int kSampMaxTiles = 4096;  // vocab <= 262144

__global__ __launch_bounds__(64 * kSampWaves) void verify_sampling_kernel(
    int K, int V, const int32_t* draft, const float* q, const float* p,
    const float* ua, const float* us, int32_t* accept, int32_t* next) {
  __shared__ double ts[kSampMaxTiles];        // tile sums
  __shared__ double seg[kSampMaxTiles / 64];  // segment sums
  __shared__ int tau_s, tile_s, mode_s;
  __shared__ double base_s, target_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int K1 = K - 1;
  if (wave == 0) {
    bool rej = false;
    if (lane < K1) {
      const int64_t o = (int64_t)b * K1 + lane;
      const int x = draft[o];
      if (x < 0 || x >= V) {
        rej = true;
      } else {
        // u * q(x) < p(x): the product of two float32 values is exact in
        // float64
        const double qx = q[o * V + x];
        const double px = p[((int64_t)b * K + lane) * V + x];
        rej = !((double)ua[o] * qx < px);
      }
    }
    const unsigned long long m = __ballot(rej);
    if (lane == 0) tau_s = m ? __ffsll((long long)m) - 1 : K1;
  }
  __syncthreads();
  const int tau = tau_s;
  const float* prow = p + ((int64_t)b * K + min(tau, K1)) * V;
  const float* qrow = q + ((int64_t)b * K1 + min(tau, K1 - 1)) * V;
  const int ntiles = (V + 63) / 64, nseg = (ntiles + 63) / 64;
  // mode 1: residual max(0, p - q) after a rejection; mode 0: p itself (all
  // accepted, or a residual that is zero everywhere)
  auto weight = [&](int mode, int i) -> double {
    if (i >= V) return 0.0;
    const double pv = prow[i];
    return mode ? fmax(pv - (double)qrow[i], 0.0) : pv;
  };
  for (int mode = tau < K1 ? 1 : 0; mode >= 0; --mode) {
    for (int t = wave; t < ntiles; t += kSampWaves) {
      double v = weight(mode, t * 64 + lane);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0) ts[t] = v;
    }
    __syncthreads();
    if (tid < nseg) {
      const int t1 = min(ntiles, tid * 64 + 64);
      double v = 0.0;
      for (int t = tid * 64; t < t1; ++t) v += ts[t];
      seg[tid] = v;
    }
    __syncthreads();
    if (tid == 0) {
      double total = 0.0;
      for (int g = 0; g < nseg; ++g) total += seg[g];
      tile_s = -1;
      if (total > 0.0) {
        const double t = (double)us[b] * total;
        double run = 0.0, base = 0.0;
        int gs = -1;
        for (int g = 0; g < nseg; ++g) {
          if (seg[g] > 0.0) {
            gs = g;
            base = run;
            if (run + seg[g] > t) break;
          }
          run += seg[g];
        }
        run = base;
        int ks = -1;
        const int t1 = min(ntiles, gs * 64 + 64);
        for (int k = gs * 64; k < t1; ++k) {
          if (ts[k] > 0.0) {
            ks = k;
            base = run;
            if (run + ts[k] > t) break;
          }
          run += ts[k];
        }
        tile_s = ks;
        mode_s = mode;
        base_s = base;
        target_s = t;
      }
    }
    __syncthreads();
    if (tile_s >= 0) break;  // uniform
  }
  if (wave != 0) return;
  if (tile_s < 0) {  // nothing to draw from
    if (lane == 0) {
      accept[b] = tau + 1;
      next[b] = -1;
    }
    return;
  }
  const double w = weight(mode_s, tile_s * 64 + lane);
  const double t = target_s;
  double run = base_s;
  int pick = -1, last = -1;
  for (int k = 0; k < 64; ++k) {
    const double wk = __shfl(w, k, 64);
    if (wk > 0.0) {
      last = k;
      if (pick < 0 && run + wk > t) pick = k;
    }
    run += wk;
  }
  if (lane == 0) {
    accept[b] = tau + 1;
    next[b] = tile_s * 64 + (pick >= 0 ? pick : last);
  }
}

}  // namespace

hipError_t launch_lm_merge(int rows, int ntiles, const Top2* part, Top2* part2,
                           hipStream_t s) {
  launch_k(lm_merge_kernel, dim3(rows * kMergeChunks), dim3(256), 0,
                     s, ntiles, part, part2);
  return hipGetLastError();
}

hipError_t launch_commit(int B, int K, int n_cap, int commit, bool last,
                         const Top2* part, int nrec, BlockState st,
                         int32_t* draft, float* conf, float* margin,
                         hipStream_t s) {
  if (K > 64 || nrec < 1) return hipErrorInvalidValue;
  launch_k(commit_kernel, dim3(B), dim3(64 * kCommitWaves), 0, s, K,
                     n_cap, commit, last ? 1 : 0, part, nrec, st, draft, conf,
                     margin);
  return hipGetLastError();
}

hipError_t launch_verify_sampling(int B, int K, int V, const int32_t* draft,
                                  const float* q, const float* p,
                                  const float* u_accept, const float* u_sample,
                                  int32_t* accept, int32_t* next,
                                  hipStream_t s) {
  if (K < 2 || K > 64 || V < 1 || (V + 63) / 64 > kSampMaxTiles)
    return hipErrorInvalidValue;
  launch_k(verify_sampling_kernel, dim3(B), dim3(64 * kSampWaves),
                     0, s, K, V, draft, q, p, u_accept, u_sample, accept,
                     next);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int K, const int32_t* draft,
                         const int32_t* target, int32_t* accept,
                         int32_t* next_anchor, hipStream_t s) {
  launch_k(verify_kernel, dim3((B + 63) / 64), dim3(64), 0, s, B, K,
                     draft, target, accept, next_anchor);
  return hipGetLastError();
}

}  // namespace dflash
