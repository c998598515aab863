// Synthetic target for tests and benchmarks (separate library): stands in
// for the target model's greedy tokens; see include/dflash_harness.h.
#include <hip/hip_runtime.h>

#include "../../include/dflash_harness.h"
#include "common.h"

namespace {

// The drafting kernels' FP8 E4M3 -> bf16 widening (dflash::fp8x8_to_bf16)
// applied to a code array, eight codes per thread.
__global__ void fp8_to_bf16_kernel(int n8, const unsigned char* codes,
                                   unsigned short* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const uint32_t* c = reinterpret_cast<const uint32_t*>(codes) + 2 * i;
  const dflash::u32x4 v = dflash::fp8x8_to_bf16(c[0], c[1]);
  *reinterpret_cast<dflash::u32x4*>(out + 8 * i) = v;
}

__global__ void synth_target_kernel(int B, int K, int V, const int32_t* draft,
                                    const float* u, const int32_t* r,
                                    const int32_t* tail, const float* p,
                                    int32_t* target) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * K) return;
  const int b = idx / K, j = idx % K;
  if (j == K - 1) {
    target[idx] = tail[b];
    return;
  }
  const int o = b * (K - 1) + j;
  const int dj = draft[o];
  target[idx] = u[o] < p[j] ? dj : (int)(((int64_t)dj + 1 + r[o]) % V);
}

// The stand-in target model, one workgroup of 4 waves per position:
//   x_0 = E[token]; x_k = bf16(RMSNorm(x_{k-1} + W_k x_{k-1}) * g_k) for the
//   n_t hooked layers; next = argmax(W_o x_{n_t}), lowest id on ties.
// A wave computes one output at a time: lanes take every 64th contraction
// element in order, then a fixed butterfly, so a position's values do not
// depend on which other positions share the launch.  Norm statistics and
// the scaling are float64 with one rounding to bf16.
constexpr int kTgtMaxHooks = 8;
struct TargetArgs {
  const void* layers[kTgtMaxHooks];
  const void* gains[kTgtMaxHooks];
  void* hooks[kTgtMaxHooks];
  int nt, Dt, V;
  int64_t ld;
  float eps;
  const int32_t* tokens;
  const void* embed;
  const void* head;
  int32_t* next;
  float* margin;
};

__device__ __forceinline__ float bf(const unsigned short* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ __forceinline__ float row_dot(const unsigned short* w,
                                         const float* x, int n, int lane) {
  float acc = 0.f;
  for (int i = lane; i < n; i += 64) acc += bf(w, i) * x[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  return acc;
}

__global__ __launch_bounds__(256) void target_kernel(TargetArgs a) {
  extern __shared__ float sm[];
  float* x = sm;           // [Dt]
  float* u = sm + a.Dt;    // [Dt]
  __shared__ double red[4];
  __shared__ float bm1[4], bm2[4];
  __shared__ int bi1[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int Dt = a.Dt;
  int tok = a.tokens[row];
  tok = min(max(tok, 0), a.V - 1);
  const unsigned short* E =
      static_cast<const unsigned short*>(a.embed) + (int64_t)tok * Dt;
  for (int j = tid; j < Dt; j += 256) x[j] = bf(E, j);
  __syncthreads();
  for (int k = 0; k < a.nt; ++k) {
    const unsigned short* W = static_cast<const unsigned short*>(a.layers[k]);
    for (int j = wave; j < Dt; j += 4) {
      const float d = row_dot(W + (int64_t)j * Dt, x, Dt, lane);
      if (lane == 0) u[j] = x[j] + d;
    }
    __syncthreads();
    double ss = 0.0;
    for (int j = tid; j < Dt; j += 256) ss += (double)u[j] * u[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double inv =
        1.0 / sqrt((red[0] + red[1] + red[2] + red[3]) / Dt + (double)a.eps);
    const unsigned short* g = static_cast<const unsigned short*>(a.gains[k]);
    unsigned short* h =
        static_cast<unsigned short*>(a.hooks[k]) + (int64_t)row * a.ld;
    for (int j = tid; j < Dt; j += 256) {
      const uint32_t b = dflash::f64_to_bf16((double)u[j] * inv * bf(g, j));
      h[j] = (unsigned short)b;
      x[j] = __uint_as_float(b << 16);
    }
    __syncthreads();
  }
  // greedy head: per wave (max, lowest index of the max, second max)
  const unsigned short* Wo = static_cast<const unsigned short*>(a.head);
  float m1 = -INFINITY, m2 = -INFINITY;
  int i1 = 0x7fffffff;
  for (int v = wave; v < a.V; v += 4) {
    const float z = row_dot(Wo + (int64_t)v * Dt, x, Dt, lane);
    if (z > m1) {
      m2 = m1;
      m1 = z;
      i1 = v;
    } else if (z > m2) {
      m2 = z;
    }
  }
  if (lane == 0) {
    bm1[wave] = m1;
    bm2[wave] = m2;
    bi1[wave] = i1;
  }
  __syncthreads();
  if (tid == 0) {
    float t1 = bm1[0], t2 = bm2[0];
    int ti = bi1[0];
    for (int w = 1; w < 4; ++w) {
      const bool wins = bm1[w] > t1 || (bm1[w] == t1 && bi1[w] < ti);
      if (wins) {
        t2 = fmaxf(t1, bm2[w]);
        t1 = bm1[w];
        ti = bi1[w];
      } else {
        t2 = fmaxf(t2, bm1[w]);
      }
    }
    a.next[row] = ti;
    if (a.margin) a.margin[row] = t1 - t2;
  }
}

// Plain streaming read: 256 KiB tiles t = wg, wg + grid, ...; each of the
// 16 waves reads its 16 KiB share of a tile as two groups of eight 1 KiB
// loads, and the groups are double-buffered across the wave's tiles (the
// next group in flight while the current one is consumed, 16 KiB per wave).
// Every address lies inside its tile.  The xor of everything read goes to
// *sink only if it equals a value it never takes in practice, so the loads
// stay.
constexpr int kProbeTile = 256 * 1024;
__global__ __launch_bounds__(1024) void read_probe_kernel(const char* buf,
                                                          int64_t ntiles,
                                                          int32_t* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t mine = blockIdx.x < ntiles
                           ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1
                           : 0;  // tiles of this workgroup
  const int64_t ngroups = 2 * mine;
  // group g: tile blockIdx.x + (g / 2) grid, half g % 2 of this wave's share
  auto group = [&](int64_t g) {
    const int64_t t = blockIdx.x + (g >> 1) * gridDim.x;
    return buf + t * kProbeTile + wave * (kProbeTile / 16) +
           (g & 1) * (kProbeTile / 32) + lane * 16;
  };
  dflash::u32x4 acc = {0u, 0u, 0u, 0u}, x[8], y[8];
  auto load = [&](dflash::u32x4(&r)[8], int64_t g) {
    const char* b = group(g);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r[j] = *reinterpret_cast<const dflash::u32x4*>(b + j * 1024);
  };
  auto use = [&](const dflash::u32x4(&r)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= r[j];
  };
  if (ngroups > 0) load(x, 0);
  for (int64_t g = 0; g < ngroups; g += 2) {
    load(y, g + 1);  // ngroups is even: group g + 1 exists
    use(x);
    if (g + 2 < ngroups) load(x, g + 2);
    use(y);
  }
  if (acc.x == 0x9E3779B9u && acc.y == 0x7F4A7C15u && acc.z == 1u) sink[0] = 1;
}

}  // namespace

extern "C" int dflash_harness_read_probe(void* stream, const void* buf,
                                         int64_t bytes, int32_t grid,
                                         int32_t* sink) {
  if (!buf || !sink || bytes < kProbeTile || bytes % kProbeTile != 0 ||
      grid < 1 || grid > 65536 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return -1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(1024), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const char*>(buf), bytes / kProbeTile, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int dflash_harness_target_forward(
    void* stream, int32_t rows, int32_t num_hooks, int32_t hidden,
    int32_t vocab, const int32_t* tokens, const void* embed,
    const void* const* layers, const void* const* gains, const void* head,
    float eps, void* const* hooks, int64_t ld, int32_t* next_token,
    float* margin) {
  if (rows < 1 || num_hooks < 1 || num_hooks > kTgtMaxHooks || hidden < 64 ||
      hidden > 4096 || vocab < 2 || ld < hidden || !tokens || !embed ||
      !layers || !gains || !head || !hooks || !next_token)
    return -1;
  TargetArgs a{};
  for (int k = 0; k < num_hooks; ++k) {
    if (!layers[k] || !gains[k] || !hooks[k]) return -1;
    a.layers[k] = layers[k];
    a.gains[k] = gains[k];
    a.hooks[k] = hooks[k];
  }
  a.nt = num_hooks;
  a.Dt = hidden;
  a.V = vocab;
  a.ld = ld;
  a.eps = eps;
  a.tokens = tokens;
  a.embed = embed;
  a.head = head;
  a.next = next_token;
  a.margin = margin;
  hipLaunchKernelGGL(target_kernel, dim3(rows), dim3(256),
                     2 * hidden * sizeof(float),
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int dflash_harness_synth_target(void* stream, int32_t batch,
                                           int32_t block_size, int32_t vocab,
                                           const int32_t* draft, const float* u,
                                           const int32_t* r, const int32_t* tail,
                                           const float* p, int32_t* target) {
  if (batch < 1 || block_size < 2 || vocab < 2 || !draft || !u || !r || !tail ||
      !p || !target)
    return -1;
  const int n = batch * block_size;
  hipLaunchKernelGGL(synth_target_kernel, dim3((n + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), batch, block_size, vocab,
                     draft, u, r, tail, p, target);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int dflash_harness_fp8_to_bf16(void* stream, int32_t n,
                                          const uint8_t* codes,
                                          uint16_t* out) {
  if (n < 8 || n % 8 != 0 || !codes || !out ||
      (reinterpret_cast<uintptr_t>(codes) & 7u) ||
      (reinterpret_cast<uintptr_t>(out) & 15u))
    return -1;
  const int n8 = n / 8;
  hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3((n8 + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), n8, codes, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
