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
