/*
 * dflash_harness.h -- test and benchmark harness kernels (libdflash_harness).
 *
 * Not part of the drafting path.  The target model is out of scope: its
 * greedy tokens are a seeded synthetic stand-in that agrees with each drafted
 * position with a chosen probability, so verification sees realistic
 * acceptance lengths.
 */
#ifndef DFLASH_HARNESS_H
#define DFLASH_HARNESS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Synthetic target greedy ids, asynchronously on `stream` (a hipStream_t).
 * For b < batch and drafted index j < K-1:
 *   target[b][j] = draft[b][j]                     if u[b][j] < p[j]
 *                = (draft[b][j] + 1 + r[b][j]) % V  otherwise (never the draft)
 * and target[b][K-1] = tail[b].
 * draft, r: [batch, K-1] int32 (r in [0, V-2]); u: [batch, K-1] fp32;
 * p: [K-1] fp32; tail: [batch] int32; target: [batch, K] int32 out.
 * All device pointers.  Returns 0 on success, -1 on a bad argument, -4 on a
 * HIP launch error. */
int dflash_harness_synth_target(void* stream, int32_t batch, int32_t block_size,
                                int32_t vocab, const int32_t* draft,
                                const float* u, const int32_t* r,
                                const int32_t* tail, const float* p,
                                int32_t* target);

/* The drafting kernels' FP8 E4M3 -> bf16 widening applied to n codes
 * (n a multiple of 8; codes 8-byte aligned, out 16-byte aligned), so a test
 * can check it on every code: out[k] = bf16 bits of value(codes[k]).
 * Returns 0, -1 on a bad argument, -4 on a HIP launch error. */
int dflash_harness_fp8_to_bf16(void* stream, int32_t n, const uint8_t* codes,
                               uint16_t* out);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_HARNESS_H */
