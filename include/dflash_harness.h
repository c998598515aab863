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

/* A small stand-in target model, for closing the speculative loop on the
 * GPU: for each of `rows` positions with token tokens[r],
 *   x_0 = embed[token]                       (bf16 [vocab][hidden])
 *   x_k = bf16(RMSNorm(x_{k-1} + layers[k-1] x_{k-1}) * gains[k-1])
 *         for k = 1 .. num_hooks             (layers bf16 [hidden][hidden],
 *                                             gains bf16 [hidden])
 *   hooks[k-1][r][:] = x_k                   (bf16, row stride ld)
 *   next_token[r] = argmax(head x_{num_hooks}), lowest id on ties
 *   margin[r] = top-1 minus top-2 logit (fp32; margin may be NULL)
 * Each position is computed by its own workgroup in a fixed order: the
 * results of a position do not depend on the other positions of the call.
 * hooks, layers, gains: HOST arrays of num_hooks DEVICE pointers.
 * 1 <= num_hooks <= 8, 64 <= hidden <= 4096, ld >= hidden.  Returns 0, -1
 * on a bad argument, -4 on a HIP launch error. */
int dflash_harness_target_forward(void* stream, int32_t rows,
                                  int32_t num_hooks, int32_t hidden,
                                  int32_t vocab, const int32_t* tokens,
                                  const void* embed, const void* const* layers,
                                  const void* const* gains, const void* head,
                                  float eps, void* const* hooks, int64_t ld,
                                  int32_t* next_token, float* margin);

/* The drafting kernels' FP8 E4M3 -> bf16 widening applied to n codes
 * (n a multiple of 8; codes 8-byte aligned, out 16-byte aligned), so a test
 * can check it on every code: out[k] = bf16 bits of value(codes[k]).
 * Returns 0, -1 on a bad argument, -4 on a HIP launch error. */
int dflash_harness_fp8_to_bf16(void* stream, int32_t n, const uint8_t* codes,
                               uint16_t* out);

/* A plain streaming read of `bytes` (a multiple of 256 KiB; buf 16-byte
 * aligned) by `grid` workgroups of 16 waves, 8 KiB per wave in flight, for
 * measuring the HBM read rate the machine delivers to a pure stream (the
 * reference for the drafting kernels' bandwidth fractions).  Nothing is
 * written except, practically never, sink[0].  Returns 0, -1 on a bad
 * argument, -4 on a HIP launch error. */
int dflash_harness_read_probe(void* stream, const void* buf, int64_t bytes,
                              int32_t grid, int32_t* sink);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_HARNESS_H */
