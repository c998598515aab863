// Per-element GEMM epilogues shared by the wide (batch-1) and tiled
// (batched) projection kernels.
#pragma once

#include "../../include/dflash.h"
#include "kernels.h"

namespace dflash {

// Rotation of one (x_i, x_{i+d/2}) pair, in float64 so that the result is
// rounded once, to the storage type.
__device__ __forceinline__ void rope_pair(double a, double b, double2 cs,
                                          double& ra, double& rb) {
  ra = a * cs.x - b * cs.y;
  rb = b * cs.x + a * cs.y;
}

// bf16 of silu(a) * b, rounded exactly as the float64 evaluation would be.
// The float evaluation (expf, one add, a correctly rounded divide, one
// multiply) is within a few float ulps of the exact value; unless that lands
// within kSiluGuard float ulps of a bf16 rounding midpoint (low 16 bits
// 0x8000), it rounds to the same bf16 as the exact value and as the float64
// evaluation.  Near a midpoint, for large |a| and for zero, denormal or
// non-finite results the float64 evaluation decides.
constexpr uint32_t kSiluGuard = 64;
// The float evaluation: true, with the bf16 in `bits`, where it decides.
__device__ __forceinline__ bool swiglu_bf16_float(float a, float b,
                                                  uint32_t& bits) {
  const float r = a / (1.f + expf(-a)) * b;
  const uint32_t u = __float_as_uint(r);
  const uint32_t lo = u & 0xFFFFu, ex = u & 0x7F800000u;
  bits = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return fabsf(a) < 64.f && ex != 0u && ex != 0x7F800000u &&
         (lo + kSiluGuard < 0x8000u || lo > 0x8000u + kSiluGuard);
}
// The float64 evaluation, for the cases the float one leaves open.
__device__ __forceinline__ uint32_t swiglu_bf16_f64(float a, float b) {
  const double da = a;
  return f64_to_bf16(da / (1.0 + exp(-da)) * (double)b);
}
__device__ __forceinline__ uint32_t swiglu_bf16(float a, float b) {
  uint32_t bits;
  return swiglu_bf16_float(a, b, bits) ? bits : swiglu_bf16_f64(a, b);
}

// One finished output pair of a MAP_PAIRS GEMM: `a` is low column `col`,
// `b` its partner at col + pair_off, both of output row `row` (< M).
//   EP_SWIGLU: act[row][col] = silu(a) * b (packed, contraction pair_off)
//   EP_QKV:    q -> RoPE -> q buffer; block k -> RoPE and v -> this layer's
//              cache at position L_b + i
//   EP_KV:     injected row -> RoPE(k), v -> cache of layer col / (2 Hkv d)
// The EP_SWIGLU element alone.
template <typename T>
__device__ __forceinline__ void swiglu_store(const GemmArgs& p, int row,
                                             int col, float a, float b) {
  T* act = static_cast<T*>(p.out_t);
  const int64_t off = packed_offset<T>(row, col, p.pair_off) / sizeof(T);
  if constexpr (sizeof(T) == 2) {
    act[off].bits = (uint16_t)swiglu_bf16(a, b);
  } else {
    const double da = a;
    store_elem(act, off, da / (1.0 + exp(-da)) * (double)b);
  }
}

template <typename T>
__device__ __forceinline__ void pair_epilogue(const GemmArgs& p, int row,
                                              int col, float a, float b) {
  if (p.ep == EP_SWIGLU) {
    swiglu_store<T>(p, row, col, a, b);
    return;
  }
  const int half = p.d / 2;
  const int head = col / p.d, i = col % p.d;  // i < d/2
  if (p.ep == EP_QKV) {
    const int bs = row / p.K;
    int L = p.ctx_len[bs];
    if (L < 0 || L > p.max_len) {
      set_error(p.err, DFLASH_DEVERR_CTX_LEN);
      L = min(max(L, 0), p.max_len);
    }
    const int pos = L + row % p.K;
    const double2 cs = p.rope[(int64_t)pos * half + i];
    double ra, rb;
    T* dst;
    if (head < p.Hq) {
      dst = static_cast<T*>(p.out_t) + (int64_t)row * p.Hq * p.d + head * p.d;
      rope_pair(a, b, cs, ra, rb);
    } else {
      const bool is_k = head < p.Hq + p.Hkv;
      const int h = is_k ? head - p.Hq : head - p.Hq - p.Hkv;
      dst = static_cast<T*>(p.kv) +
            (is_k ? 0 : kv_plane_rows(p.pages, p.max_batch, p.Hkv, p.P) * p.d) +
            kv_row(p.pages, p.P, p.Hkv, bs, h, pos, p.err) * p.d;
      if (is_k) {
        rope_pair(a, b, cs, ra, rb);
      } else {
        ra = a;
        rb = b;
      }
    }
    store_elem(dst, i, ra);
    store_elem(dst, i + half, rb);
    return;
  }
  // EP_KV: injected context rows
  const int seq = p.row_seq[row], pos = p.row_pos[row];
  if (seq < 0 || seq >= p.max_batch) {
    set_error(p.err, DFLASH_DEVERR_SLOT);
    return;
  }
  if (pos < 0 || pos >= p.max_ctx) {
    set_error(p.err, DFLASH_DEVERR_POS);
    return;
  }
  const int l = head / (2 * p.Hkv), w = head % (2 * p.Hkv);
  const bool is_k = w < p.Hkv;
  const int h = is_k ? w : w - p.Hkv;
  const int64_t plane =
      kv_plane_rows(p.pages, p.max_batch, p.Hkv, p.P) * p.d;
  T* dst = static_cast<T*>(p.kv) + (2 * l + (is_k ? 0 : 1)) * plane +
           kv_row(p.pages, p.P, p.Hkv, seq, h, pos, p.err) * p.d;
  double ra = a, rb = b;
  if (is_k) rope_pair(a, b, p.rope[(int64_t)pos * half + i], ra, rb);
  store_elem(dst, i, ra);
  store_elem(dst, i + half, rb);
}

// Eight consecutive finished output pairs of a bf16 MAP_PAIRS GEMM: a[k] is
// low column col + k, b[k] its partner (col % 8 == 0, the eight never cross
// a head or a 16-byte output chunk).  The arithmetic and the rounding of each
// element are those of pair_epilogue; the stores are whole 16-byte chunks.
__device__ __forceinline__ void pair_epilogue8(const GemmArgs& p, int row,
                                               int col, const float (&a)[8],
                                               const float (&b)[8]) {
  if (p.ep == EP_SWIGLU) {
    u32x4 w;
    uint16_t* wt = reinterpret_cast<uint16_t*>(&w);
#pragma unroll
    for (int k = 0; k < 8; ++k) wt[k] = (uint16_t)swiglu_bf16(a[k], b[k]);
    *reinterpret_cast<u32x4*>(static_cast<char*>(p.out_t) +
                              packed_offset<bf16_t>(row, col, p.pair_off)) = w;
    return;
  }
  const int half = p.d / 2;
  const int head = col / p.d, i = col % p.d;  // i + 7 < d/2
  bool rot = true;
  int pos;
  bf16_t* dst;
  if (p.ep == EP_QKV) {
    const int bs = row / p.K;
    int L = p.ctx_len[bs];
    if (L < 0 || L > p.max_len) {
      set_error(p.err, DFLASH_DEVERR_CTX_LEN);
      L = min(max(L, 0), p.max_len);
    }
    pos = L + row % p.K;
    if (head < p.Hq) {
      dst = static_cast<bf16_t*>(p.out_t) + (int64_t)row * p.Hq * p.d +
            head * p.d;
    } else {
      const bool is_k = head < p.Hq + p.Hkv;
      const int h = is_k ? head - p.Hq : head - p.Hq - p.Hkv;
      dst = static_cast<bf16_t*>(p.kv) +
            (is_k ? 0 : kv_plane_rows(p.pages, p.max_batch, p.Hkv, p.P) * p.d) +
            kv_row(p.pages, p.P, p.Hkv, bs, h, pos, p.err) * p.d;
      rot = is_k;
    }
  } else {  // EP_KV: injected context rows
    const int seq = p.row_seq[row];
    pos = p.row_pos[row];
    if (seq < 0 || seq >= p.max_batch) {
      set_error(p.err, DFLASH_DEVERR_SLOT);
      return;
    }
    if (pos < 0 || pos >= p.max_ctx) {
      set_error(p.err, DFLASH_DEVERR_POS);
      return;
    }
    const int l = head / (2 * p.Hkv), w = head % (2 * p.Hkv);
    const bool is_k = w < p.Hkv;
    const int h = is_k ? w : w - p.Hkv;
    const int64_t plane =
        kv_plane_rows(p.pages, p.max_batch, p.Hkv, p.P) * p.d;
    dst = static_cast<bf16_t*>(p.kv) + (2 * l + (is_k ? 0 : 1)) * plane +
          kv_row(p.pages, p.P, p.Hkv, seq, h, pos, p.err) * p.d;
    rot = is_k;
  }
  u32x4 wa, wb;
  bf16_t* ta = reinterpret_cast<bf16_t*>(&wa);
  bf16_t* tb = reinterpret_cast<bf16_t*>(&wb);
  const double2* cs = p.rope + (int64_t)pos * half + i;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    double ra = a[k], rb = b[k];
    if (rot) rope_pair(a[k], b[k], cs[k], ra, rb);
    store_elem(ta, k, ra);
    store_elem(tb, k, rb);
  }
  *reinterpret_cast<u32x4*>(dst + i) = wa;
  *reinterpret_cast<u32x4*>(dst + i + half) = wb;
}

// Debug copy of one LM-head logit (row -> block row via the row map).
__device__ __forceinline__ void store_debug_logit(const GemmArgs& p, int row,
                                                  int col, float z) {
  const int br = p.rowmap[row];
  if (br >= 0)
    p.logits[((int64_t)(br / p.K) * (p.K - 1) + (br % p.K) - 1) * p.logits_ld +
             col] = z;
}

}  // namespace dflash
