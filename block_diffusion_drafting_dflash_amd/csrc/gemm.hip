// Skinny MFMA GEMMs for the drafter's projections and its LM head.
//
// The drafter multiplies 16 * batch block rows (or the injected context rows)
// by weight matrices stored [out, in].  At batch 1 the job is streaming each
// weight byte from HBM exactly once, so a workgroup owns 64 output columns
// (four 16-column MFMA tiles) and its four waves split the contraction,
// interleaved by 32-element steps so that together they read each weight
// row contiguously.  The waves' partial tiles are summed through LDS in a
// fixed order; a grid-z split of the contraction adds workgroups when the
// output is narrow, and the epilogue kernels sum those slices in order.
//
// Fragment layout (both operands K-contiguous in memory): lane l loads 16
// bytes of row / column l % 16 at contraction offset (l / 16) * E within the
// current step, which is the same slot on both operands, so any intra-
// instruction contraction order of the MFMA gives the same sum.
#include "kernels.h"

namespace dflash {

namespace {

template <typename T, int MT, int NT>
__device__ __forceinline__ void gemm_core(const GemmArgs& p, int n_base,
                                          int m_base, int k_lo, int k_hi,
                                          f32x4 (&acc)[MT][NT]) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC;
  constexpr int STEP = 4 * KC;  // the four waves interleave by KC
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;

  const char* bptr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = min(n_base + 16 * t + r, p.N - 1);
    int s = 0;
    while (s + 1 < p.b_nseg && n >= p.b_n0[s + 1]) ++s;
    bptr[t] = static_cast<const char*>(p.b_ptr[s]) +
              ((int64_t)(n - p.b_n0[s]) * p.Kd + g * E) * (int64_t)sizeof(T);
  }
  int64_t aoff[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = min(m_base + 16 * m + r, p.M - 1);
    aoff[m] = ((int64_t)row * p.lda + g * E) * (int64_t)sizeof(T);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int seg = k_lo / p.a_seg_k; seg * p.a_seg_k < k_hi; ++seg) {
    const int s0 = seg * p.a_seg_k;
    const int ks = max(k_lo, s0), ke = min(k_hi, s0 + p.a_seg_k);
    const char* abase = static_cast<const char*>(p.a_ptr[seg]) -
                        (int64_t)s0 * (int64_t)sizeof(T);
    int kc = ks + wave * KC;
    constexpr int U = 4;
    for (; kc + (U - 1) * STEP < ke; kc += U * STEP) {
      u32x4 bf[U][NT], af[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          bf[u][t] = load16(bptr[t] + (int64_t)(kc + u * STEP) * sizeof(T));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          af[u][m] = load16(abase + aoff[m] +
                            (int64_t)(kc + u * STEP) * sizeof(T));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int t = 0; t < NT; ++t) mma16(acc[m][t], af[u][m], bf[u][t], T());
    }
    for (; kc < ke; kc += STEP) {
      u32x4 bf[NT], af[MT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        bf[t] = load16(bptr[t] + (int64_t)kc * sizeof(T));
#pragma unroll
      for (int m = 0; m < MT; ++m)
        af[m] = load16(abase + aoff[m] + (int64_t)kc * sizeof(T));
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) mma16(acc[m][t], af[m], bf[t], T());
    }
  }
}

// Each wave parks its tile in LDS: red[wave][(m*NT + t)*4 + j][lane].
template <int MT, int NT>
__device__ __forceinline__ void park(const f32x4 (&acc)[MT][NT], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[((wave * MT * NT + m * NT + t) * 4 + j) * 64 + lane] = acc[m][t][j];
  __syncthreads();
}

template <typename T, int MT, int NT>
__global__ __launch_bounds__(256) void gemm_partial_kernel(GemmArgs p) {
  __shared__ float red[4 * MT * NT * 4 * 64];
  const int n_base = blockIdx.x * 16 * NT, m_base = blockIdx.y * 16 * MT;
  const int k_lo = blockIdx.z * p.k_split;
  const int k_hi = min(p.Kd, k_lo + p.k_split);
  f32x4 acc[MT][NT];
  gemm_core<T, MT, NT>(p, n_base, m_base, k_lo, k_hi, acc);
  park<MT, NT>(acc, red);
  constexpr int S = MT * NT * 4 * 64;
  float* out = p.out + (int64_t)blockIdx.z * p.M * p.N;
  for (int idx = threadIdx.x; idx < S; idx += 256) {
    const float v = red[idx] + red[S + idx] + red[2 * S + idx] + red[3 * S + idx];
    const int e = idx >> 6, ln = idx & 63;
    const int j = e & 3, mt = (e >> 2) / NT, t = (e >> 2) % NT;
    const int row = m_base + 16 * mt + 4 * (ln >> 4) + j;
    const int col = n_base + 16 * t + (ln & 15);
    if (row < p.M && col < p.N) out[(int64_t)row * p.N + col] = v;
  }
}

// LM head: z = A . W^T for a 64-column vocabulary tile, reduced per row to
// (max, argmax, 2nd max, sum exp(z - max)) without writing logits (unless a
// debug buffer is given).
template <typename T, int MT>
__global__ __launch_bounds__(256) void lmhead_kernel(GemmArgs p, Top2* part,
                                                     float* logits,
                                                     const int* rowmap,
                                                     int64_t logits_ld) {
  constexpr int NT = 4;
  __shared__ float red[4 * MT * NT * 4 * 64];
  const int n_base = blockIdx.x * 64, m_base = blockIdx.y * 16 * MT;
  f32x4 acc[MT][NT];
  gemm_core<T, MT, NT>(p, n_base, m_base, 0, p.Kd, acc);
  park<MT, NT>(acc, red);
  constexpr int S = MT * NT * 4 * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = n_base + lane;
  const int t = lane >> 4;
  for (int rr = wave; rr < 16 * MT; rr += 4) {
    const int row = m_base + rr;
    if (row >= p.M) break;
    const int mt = rr >> 4, j = rr & 3;
    const int ln = ((rr & 15) >> 2) * 16 + (lane & 15);
    const int idx = ((mt * NT + t) * 4 + j) * 64 + ln;
    const float z = red[idx] + red[S + idx] + red[2 * S + idx] + red[3 * S + idx];
    Top2 v = top2_empty();
    if (col < p.N) {
      v.m1 = z;
      v.i1 = col;
      v.s = 1.f;
      if (logits != nullptr) {
        const int dst = rowmap[row];
        if (dst >= 0) logits[(int64_t)dst * logits_ld + col] = z;
      }
    }
    v = top2_wave(v);
    if (lane == 0) part[(int64_t)row * gridDim.x + blockIdx.x] = v;
  }
}

template <typename T>
hipError_t launch_gemm_t(const GemmPlan& pl, const GemmArgs& a, hipStream_t s) {
  dim3 grid(pl.gx, pl.gy, pl.gz), block(256);
  switch (pl.MT) {
    case 1: hipLaunchKernelGGL((gemm_partial_kernel<T, 1, kGemmNT>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_partial_kernel<T, 2, kGemmNT>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_partial_kernel<T, 4, kGemmNT>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_lmhead_t(const GemmPlan& pl, const GemmArgs& a, Top2* part,
                           float* logits, const int* rowmap, int64_t ld,
                           hipStream_t s) {
  dim3 grid(pl.gx, pl.gy, 1), block(256);
  switch (pl.MT) {
    case 1: hipLaunchKernelGGL((lmhead_kernel<T, 1>), grid, block, 0, s, a, part, logits, rowmap, ld); break;
    case 2: hipLaunchKernelGGL((lmhead_kernel<T, 2>), grid, block, 0, s, a, part, logits, rowmap, ld); break;
    case 4: hipLaunchKernelGGL((lmhead_kernel<T, 4>), grid, block, 0, s, a, part, logits, rowmap, ld); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int pick_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

}  // namespace

GemmPlan plan_gemm(int M, int N, int Kd, bool bf16, int num_cu) {
  const int KC = bf16 ? Storage<bf16_t>::KC : Storage<float>::KC;
  GemmPlan pl;
  pl.MT = pick_mt(M);
  pl.gx = (N + 16 * kGemmNT - 1) / (16 * kGemmNT);
  pl.gy = (M + 16 * pl.MT - 1) / (16 * pl.MT);
  const int chunks = Kd / KC;
  const int base = pl.gx * pl.gy;
  const int target = 4 * num_cu;
  // at least four steps per wave in every slice
  const int max_split = chunks / 16 > 1 ? chunks / 16 : 1;
  int gz = (target + base - 1) / base;
  if (gz > max_split) gz = max_split;
  if (gz < 1) gz = 1;
  const int per = (chunks + gz - 1) / gz;
  pl.k_split = per * KC;
  pl.gz = (Kd + pl.k_split - 1) / pl.k_split;
  pl.partial_floats = (size_t)pl.gz * M * N;
  return pl;
}

GemmPlan plan_lmhead(int M, int N, int Kd, bool bf16) {
  GemmPlan pl;
  pl.MT = pick_mt(M);
  pl.gx = (N + 63) / 64;
  pl.gy = (M + 16 * pl.MT - 1) / (16 * pl.MT);
  pl.gz = 1;
  pl.k_split = Kd;
  pl.partial_floats = 0;
  (void)bf16;
  return pl;
}

hipError_t launch_gemm(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                       hipStream_t s) {
  return bf16 ? launch_gemm_t<bf16_t>(pl, a, s) : launch_gemm_t<float>(pl, a, s);
}

hipError_t launch_lmhead(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                         Top2* part, float* logits, const int* rowmap,
                         int64_t logits_ld, hipStream_t s) {
  return bf16 ? launch_lmhead_t<bf16_t>(pl, a, part, logits, rowmap, logits_ld, s)
              : launch_lmhead_t<float>(pl, a, part, logits, rowmap, logits_ld, s);
}

}  // namespace dflash
