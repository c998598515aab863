// Synthetic target for tests and benchmarks (separate library): stands in
// for the target model's greedy tokens; see include/dflash_harness.h.
#include <hip/hip_runtime.h>

#include "../../include/dflash_harness.h"

namespace {

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

}  // namespace

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
