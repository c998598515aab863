// Shared device helpers for the DFlash gfx950 kernels: storage types, 16-byte
// fragment loads, the MFMA step, and wave-level shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage tag for bf16 tensors (bits held in a uint16).
struct bf16_t {
  uint16_t bits;
};

template <typename T> struct Storage;

// One lane fragment is 16 bytes.  E = elements per fragment; KC = elements of
// the contraction covered by one fragment across the four 16-lane groups of a
// wave (the step of the K loop).
template <> struct Storage<bf16_t> {
  static constexpr int E = 8;
  static constexpr int KC = 32;
};
template <> struct Storage<float> {
  static constexpr int E = 4;
  static constexpr int KC = 16;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Round a float64 value to the nearest bf16, ties to even, in one rounding:
// float64 -> float32 rounded to odd (toward zero, then the last bit set if
// anything was discarded), then to bf16 nearest-even; the intermediate has
// more than two extra bits, so the result equals a direct rounding.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
  const float f = __double2float_rz(v);
  uint32_t u = __float_as_uint(f);
  if ((double)f != v) u |= 1u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float load_elem(const bf16_t* p, int64_t i) {
  return bf16_to_f32(p[i].bits);
}
__device__ __forceinline__ float load_elem(const float* p, int64_t i) {
  return p[i];
}
__device__ __forceinline__ void store_elem(bf16_t* p, int64_t i, float v) {
  p[i].bits = (uint16_t)f32_to_bf16(v);
}
__device__ __forceinline__ void store_elem(float* p, int64_t i, float v) {
  p[i] = v;
}
__device__ __forceinline__ void store_elem(bf16_t* p, int64_t i, double v) {
  p[i].bits = (uint16_t)f64_to_bf16(v);
}
__device__ __forceinline__ void store_elem(float* p, int64_t i, double v) {
  p[i] = (float)v;
}
// Value after rounding to the storage type (what a store then load returns).
__device__ __forceinline__ float round_to(bf16_t, float v) {
  return bf16_to_f32(f32_to_bf16(v));
}
__device__ __forceinline__ float round_to(float, float v) { return v; }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// acc += A_frag . B_frag over one fragment step.  Lane l supplies row (A) or
// column (B) l % 16 and contraction slots of lane group l / 16; the two
// operands must place the same contraction index in the same (lane group,
// element) slot.  Output: lane l, register j holds row 4*(l/16)+j, column
// l % 16.
__device__ __forceinline__ void mma16(f32x4& acc, u32x4 a, u32x4 b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0,
      0);
}
__device__ __forceinline__ void mma16(f32x4& acc, u32x4 a, u32x4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x),
                                             __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y),
                                             __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z),
                                             __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w),
                                             __uint_as_float(b.w), acc, 0, 0, 0);
}

// 32x32 output tile, contraction 16 (bf16).  Lane l supplies row (A) or
// column (B) l % 32 with contraction elements 8*(l/32) .. +8; register j of
// the result holds row 8*(j/4) + 4*(l/32) + j%4, column l % 32 (checked on
// gfx950 against a host product).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void mma32(f32x16& acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0,
      0);
}

// Eight FP8 E4M3 values (the 8 bytes of lo, hi in memory order) widened to
// one 16-byte bf16 fragment, element k from byte k.  Every E4M3 value is a
// bf16 value (3 of bf16's 7 mantissa bits, exponents well inside its range),
// so the conversion is exact; the per-row scale is applied to the sums.
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r.x = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

// Prefetch loads of pipelined loops are issued as inline assembly, so that
// the compiler's wait insertion (which drains every outstanding load at a
// loop header or a branch) does not see them; the loop waits for exactly the
// loads it needs with vm_wait<N>, tied to the register it is about to read.
// Every such load is waited for (vm_wait<0>) before its register can be
// reused or the wave ends.
__device__ __forceinline__ u32x4 stage_load(const void* p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}
template <int N>
__device__ __forceinline__ void vm_wait(u32x4& v) {
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(v) : "n"(N));
}


// Waits for registers st[0 .. LIM) of one batch of staging loads, issued in
// that order, with AHEAD further loads issued after the batch: register I
// is complete once at most AHEAD + LIM - 1 - I loads are outstanding.
template <int I, int LIM, int AHEAD>
__device__ __forceinline__ void stage_wait(u32x4* st) {
  if constexpr (I < LIM) {
    vm_wait<AHEAD + LIM - 1 - I>(st[I]);
    stage_wait<I + 1, LIM, AHEAD>(st);
  }
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x == 64 * nwaves (nwaves <= 16), fixed order.
template <int NWAVES, typename F>
__device__ __forceinline__ F block_sum(F v, F* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  F t = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

// Running (max, argmax, second max, sum of exp(z - max)) over a set of
// logits.  Merging is associative and commutative in exact arithmetic for
// everything but the floating-point sum, which callers merge in a fixed
// order.  Ties in the maximum go to the lower index.
struct Top2 {
  float m1;
  int i1;
  float m2;
  float s;
};

__device__ __forceinline__ Top2 top2_empty() {
  Top2 t;
  t.m1 = -INFINITY;
  t.i1 = 0x7fffffff;
  t.m2 = -INFINITY;
  t.s = 0.f;
  return t;
}

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  const bool b_wins = (b.m1 > a.m1) || (b.m1 == a.m1 && b.i1 < a.i1);
  Top2 w = b_wins ? b : a;
  Top2 l = b_wins ? a : b;
  Top2 r;
  r.m1 = w.m1;
  r.i1 = w.i1;
  r.m2 = fmaxf(w.m2, l.m1);
  const float sl = (l.m1 == -INFINITY) ? 0.f : l.s * __expf(l.m1 - w.m1);
  r.s = w.s + sl;
  return r;
}

__device__ __forceinline__ Top2 top2_shfl_xor(Top2 t, int o) {
  Top2 r;
  r.m1 = __shfl_xor(t.m1, o, 64);
  r.i1 = __shfl_xor(t.i1, o, 64);
  r.m2 = __shfl_xor(t.m2, o, 64);
  r.s = __shfl_xor(t.s, o, 64);
  return r;
}

// Butterfly merge across the 64 lanes; every lane ends with the result.
// The butterfly pairs differ per lane, so the float sum is only guaranteed
// identical on a lane-by-lane basis run to run: callers read lane 0.
__device__ __forceinline__ Top2 top2_wave(Top2 t) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) t = top2_merge(t, top2_shfl_xor(t, o));
  return t;
}

__device__ __forceinline__ void set_error(int* err, int bit) {
  atomicOr(err, bit);
}

}  // namespace dflash
