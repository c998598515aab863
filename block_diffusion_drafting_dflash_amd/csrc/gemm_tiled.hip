// MFMA GEMMs for the batched drafter: 64 to a few thousand rows, where the
// projections and the LM head are dense contractions rather than weight
// streams (bf16).
//
// A workgroup of WM x WN waves owns a (32 WM TM) x (32 WN TN) output block
// over the whole contraction; each wave owns TM x TN tiles of 32 x 32 and
// runs the 32x32x16 MFMA (on gfx950 it has twice the throughput of the
// 16x16x32 form).  Operands are packed fragment-major (1 KiB per 16 rows x
// one 32-wide contraction step), so staging a step into LDS is one
// contiguous 1 KiB load per fragment; a 32-row MFMA operand is read back as
// 16 bytes per lane from two fragments.  PD steps are kept in flight in
// registers ahead of the double-buffered LDS stage the MFMAs read, with one
// barrier per step.  Each wave applies the epilogue to its own tiles
// straight from the accumulators (partner columns for RoPE and SwiGLU come
// from the lane 8 apart), so the block never round-trips its output through
// LDS.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the mapping below
// gives the row blocks of one column block workgroup ids 8 apart, so they
// run on the same XCD and read that weight block through one L2.
#include "gemm_epilogue.h"

namespace dflash {

namespace {

// Epilogue of one 32 x 32 accumulator tile: rows row0.., 16-column tiles
// ctile and ctile + 1 (lanes 16-31 of each half-wave take the second).
__device__ __forceinline__ void tile_epilogue(const GemmArgs& p, int row0,
                                              int ctile, const f32x16& acc,
                                              int lane) {
  const int c = lane & 15;
  const int tile = ctile + ((lane >> 4) & 1);
  const bool tile_ok = tile < p.N / 16;
  const int rbase = row0 + 4 * (lane >> 5);
  if (p.ep == EP_STORE || p.ep == EP_RESID) {
    if (!tile_ok) return;
    const int col = map_col(p.cmap, p.pair_group, p.pair_off, tile, c);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = rbase + 8 * (j >> 2) + (j & 3);
      if (row < p.M) {
        float* o = p.out_f32 + (int64_t)row * p.ldo + col;
        *o = p.ep == EP_RESID ? *o + acc[j] : acc[j];
      }
    }
    return;
  }
  if (p.ep == EP_TOP2) {
    const int col = tile * 16 + c;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = rbase + 8 * (j >> 2) + (j & 3);
      Top2 v = top2_empty();
      if (row < p.M && tile_ok) {
        v.m1 = acc[j];
        v.i1 = col;
        v.s = 1.f;
        if (p.logits != nullptr) store_debug_logit(p, row, col, acc[j]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v = top2_merge(v, top2_shfl_xor(v, o));
      if (c == 0 && row < p.M && tile_ok)
        p.top2[(int64_t)row * (p.N / 16) + tile] = v;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float partner = __shfl_xor(acc[j], 8, 64);
    const int row = rbase + 8 * (j >> 2) + (j & 3);
    if (c < 8 && row < p.M && tile_ok)
      pair_epilogue<bf16_t>(
          p, row, map_col(p.cmap, p.pair_group, p.pair_off, tile, c), acc[j],
          partner);
  }
}

template <int TM, int TN, int WM, int WN>
struct Tiled {
  static constexpr int NW = WM * WN;
  static constexpr int BMT = 2 * WM * TM;  // 16-row fragments per block
  static constexpr int BNT = 2 * WN * TN;  // 16-column fragments per block
  static constexpr int NF = BMT + BNT;     // fragments per contraction step
  static constexpr int LPW = NF / NW;      // fragment loads per wave per step
  static_assert(NF % NW == 0, "fragments must split evenly over the waves");
};

// One LDS stage = SK contraction steps, multiplied from LDS buffer `cur`
// (published during the previous stage).  After the first half-step's MFMAs
// the staged registers of the next stage (loaded PD stages ago: the PD - 1
// later stages' loads may still be in flight) are waited for and published
// into the other buffer `nxt` while the remaining MFMAs run; one barrier
// then makes them visible and frees `cur`, and the same registers are
// refilled PD stages ahead.  The refill is unconditional (clamped to the last
// stage), so the loop is straight-line code.
template <int TM, int TN, int WM, int WN, int SK, int PD>
__device__ __forceinline__ void tiled_stage(
    int refill, u32x4 (&st)[Tiled<TM, TN, WM, WN>::LPW * SK],
    const char* const (&src)[Tiled<TM, TN, WM, WN>::LPW], const u32x4* cur,
    u32x4* nxt, int wave, int lane, int a_off, int w_off,
    f32x16 (&acc)[TM][TN]) {
  using C = Tiled<TM, TN, WM, WN>;
  constexpr int NL = C::LPW * SK;  // loads per stage per lane
  // step k, half h: contraction 32k + 16h .. + 16
#pragma unroll
  for (int k = 0; k < SK; ++k)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 a[TM], w[TN];
#pragma unroll
      for (int m = 0; m < TM; ++m)
        a[m] = cur[k * C::NF * 64 + a_off + m * 128 + 32 * h];
#pragma unroll
      for (int n = 0; n < TN; ++n)
        w[n] = cur[k * C::NF * 64 + w_off + n * 128 + 32 * h];
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) mma32(acc[m][n], a[m], w[n]);
      if (k == 0 && h == 0) {
        stage_wait<0, NL, (PD - 1) * NL>(st);
#pragma unroll
        for (int kk = 0; kk < SK; ++kk)
#pragma unroll
          for (int i = 0; i < C::LPW; ++i)
            nxt[(kk * C::NF + wave + i * C::NW) * 64 + lane] =
                st[kk * C::LPW + i];
      }
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < SK; ++k)
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      st[k * C::LPW + i] =
          stage_load(src[i] + ((int64_t)refill * SK + k) * 1024);
  __builtin_amdgcn_sched_barrier(0);
}

template <int TM, int TN, int WM, int WN, int SK, int PD>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(GemmArgs p,
                                                                  int gm,
                                                                  int nbn) {
  using C = Tiled<TM, TN, WM, WN>;
  __shared__ u32x4 lds[2 * SK * C::NF * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = blockIdx.x, xcd = b & 7, k = b >> 3;
  const int mb = k % gm, nb = (k / gm) * 8 + xcd;
  if (nb >= nbn) return;  // whole workgroup: padding of the XCD mapping
  const int nsteps = p.Kd / Storage<bf16_t>::KC;
  const int nstages = nsteps / SK;
  const int mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
  const int wm = wave / WN, wn = wave % WN;

  // fragment f of a step: row tile mb*BMT + f of A, else column tile
  // nb*BNT + f - BMT of W (clamped; clamped tiles are never stored)
  const char* src[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int f = wave + i * C::NW;
    int t;
    const char* base;
    if (f < C::BMT) {
      t = min(mb * C::BMT + f, mtiles - 1);
      base = static_cast<const char*>(p.a_ptr[0]);
    } else {
      t = min(nb * C::BNT + f - C::BMT, ntiles - 1);
      base = static_cast<const char*>(p.w);
    }
    src[i] = base + ((int64_t)t * nsteps * 64 + lane) * 16;
  }
  // this lane's 16 bytes of a 32-row operand: fragment (lane / 16) % 2 of
  // the pair, contraction group 2h + lane / 32, row lane % 16
  const int lo = ((lane >> 4) & 1) * 64 + (lane >> 5) * 16 + (lane & 15);
  const int a_off = wm * TM * 128 + lo;
  const int w_off = (C::BMT + wn * TN * 2) * 64 + lo;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][n][j] = 0.f;

  constexpr int NL = C::LPW * SK;
  u32x4 st[PD][NL];
#pragma unroll
  for (int j = 0; j < PD; ++j)
#pragma unroll
    for (int kk = 0; kk < SK; ++kk)
#pragma unroll
      for (int i = 0; i < C::LPW; ++i)
        st[j][kk * C::LPW + i] = stage_load(
            src[i] + ((int64_t)min(j, nstages - 1) * SK + kk) * 1024);
  // stage 0 into buffer 0; its registers then take stage PD
  stage_wait<0, NL, (PD - 1) * NL>(st[0]);
#pragma unroll
  for (int kk = 0; kk < SK; ++kk)
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      lds[(kk * C::NF + wave + i * C::NW) * 64 + lane] = st[0][kk * C::LPW + i];
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < SK; ++kk)
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      st[0][kk * C::LPW + i] = stage_load(
          src[i] + ((int64_t)min(PD, nstages - 1) * SK + kk) * 1024);
  // stage s is multiplied from buffer s % 2 while stage s + 1 (register set
  // (s + 1) % PD) is published into the other; nstages is a multiple of PD
  for (int s = 0; s < nstages; s += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j)
      tiled_stage<TM, TN, WM, WN, SK, PD>(
          min(s + j + 1 + PD, nstages - 1), st[(j + 1) % PD], src,
          lds + ((s + j) & 1) * SK * C::NF * 64,
          lds + ((s + j + 1) & 1) * SK * C::NF * 64, wave, lane, a_off, w_off,
          acc);
  }
  // the last PD stages' refills (clamped repeats) are still in flight
#pragma unroll
  for (int j = 0; j < PD; ++j)
#pragma unroll
    for (int i = 0; i < NL; ++i) vm_wait<0>(st[j][i]);

  // One copy of the epilogue code in a rolled loop; each tile is selected
  // out of the accumulators with compile-time indices (a dynamic index would
  // move the whole accumulator array to scratch memory).
#pragma unroll 1
  for (int t = 0; t < TM * TN; ++t) {
    const int m = t / TN, n = t % TN;
    const int row0 = (mb * C::BMT + (wm * TM + m) * 2) * 16;
    const int ctile = nb * C::BNT + (wn * TN + n) * 2;
    f32x16 v = acc[0][0];
#pragma unroll
    for (int mm = 0; mm < TM; ++mm)
#pragma unroll
      for (int nn = 0; nn < TN; ++nn)
        if (t == mm * TN + nn) v = acc[mm][nn];
    if (ctile < ntiles && row0 < p.M) tile_epilogue(p, row0, ctile, v, lane);
  }
}

// Direct-to-LDS form.  Each wave's fragment loads go from global memory
// straight into a ring of NBUF contraction steps in LDS (no staging
// registers, no LDS stores), so NBUF - 1 steps are in flight per workgroup.
// The load is inline assembly: the compiler's wait insertion would drain
// every in-flight load before each LDS read.  m0 carries the fragment's LDS
// byte address and lane l's 16 bytes land at m0 + 16 l, which is the packed
// fragment layout itself; nothing else in these kernels uses m0.
__device__ __forceinline__ void lds_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait_n() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// The ring holds steps s + 1 .. s + NBUF while step s is multiplied: step s
// is multiplied from registers read out of the ring one step earlier, so the
// LDS reads of step s + 1 overlap the MFMAs of step s.  Iteration s waits
// until this wave's loads of step s + 1 have landed (later steps may still
// be in flight), one barrier (every wave's part of step s + 1 is visible and
// every wave has read step s), refills step s's slot with step s + NBUF,
// reads step s + 1 and multiplies step s.
template <int TM, int TN, int WM, int WN, int NBUF>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs p,
                                                                int gm,
                                                                int nbn) {
  using C = Tiled<TM, TN, WM, WN>;
  constexpr int STAGE = C::NF * 64;  // u32x4 per contraction step
  __shared__ u32x4 lds[NBUF * STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x, xcd = b & 7, k = b >> 3;
  const int mb = k % gm, nb = (k / gm) * 8 + xcd;
  if (nb >= nbn) return;  // whole workgroup: padding of the XCD mapping
  const int nsteps = p.Kd / Storage<bf16_t>::KC;
  const int mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
  const int wm = wave / WN, wn = wave % WN;

  // fragment f = wave + i NW of a step, as in gemm_tiled_kernel
  const char* src[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int f = wave + i * C::NW;
    int t;
    const char* base;
    if (f < C::BMT) {
      t = min(mb * C::BMT + f, mtiles - 1);
      base = static_cast<const char*>(p.a_ptr[0]);
    } else {
      t = min(nb * C::BNT + f - C::BMT, ntiles - 1);
      base = static_cast<const char*>(p.w);
    }
    src[i] = base + ((int64_t)t * nsteps * 64 + lane) * 16;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(
      __attribute__((address_space(3))) void*)lds;
  // step `step` (clamped: repeats past the end are never multiplied) into
  // ring slot `slot`
  auto issue = [&](int step, int slot) {
    const int64_t off = (int64_t)min(step, nsteps - 1) * 1024;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i)
      lds_load16(src[i] + off,
                 lds0 + (uint32_t)((slot * C::NF + wave + i * C::NW) * 1024));
  };
  const int lo = ((lane >> 4) & 1) * 64 + (lane >> 5) * 16 + (lane & 15);
  const int a_off = wm * TM * 128 + lo;
  const int w_off = (C::BMT + wn * TN * 2) * 64 + lo;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][n][j] = 0.f;

  // operands of one step: A then W fragments of both half-steps
  using Ops = u32x4[2 * (TM + TN)];
  auto read = [&](Ops& r, int slot) {
    const u32x4* cur = lds + slot * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int m = 0; m < TM; ++m)
        r[h * (TM + TN) + m] = cur[a_off + m * 128 + 32 * h];
#pragma unroll
      for (int n = 0; n < TN; ++n)
        r[h * (TM + TN) + TM + n] = cur[w_off + n * 128 + 32 * h];
    }
  };
  auto mul = [&](const Ops& r) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
          mma32(acc[m][n], r[h * (TM + TN) + m], r[h * (TM + TN) + TM + n]);
  };
  // one iteration; r_now holds step s, r_next receives step s + 1
  auto iter = [&](int s, const Ops& r_now, Ops& r_next) {
    vm_wait_n<(NBUF - 2) * C::LPW>();
    __syncthreads();
    issue(s + NBUF, s % NBUF);
    read(r_next, (s + 1) % NBUF);
    // keep the reads of step s + 1 ahead of the MFMAs of step s
    __builtin_amdgcn_sched_barrier(0);
    mul(r_now);
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int j = 0; j < NBUF; ++j) issue(j, j);
  Ops r0, r1;
  vm_wait_n<(NBUF - 1) * C::LPW>();
  __syncthreads();
  read(r0, 0);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    iter(s, r0, r1);
    iter(s + 1, r1, r0);
  }
  if (s < nsteps) mul(r0);  // odd step count: the last step
  vm_wait_n<0>();  // the clamped refills past the last step

#pragma unroll 1
  for (int t = 0; t < TM * TN; ++t) {
    const int m = t / TN, n = t % TN;
    const int row0 = (mb * C::BMT + (wm * TM + m) * 2) * 16;
    const int ctile = nb * C::BNT + (wn * TN + n) * 2;
    f32x16 v = acc[0][0];
#pragma unroll
    for (int mm = 0; mm < TM; ++mm)
#pragma unroll
      for (int nn = 0; nn < TN; ++nn)
        if (t == mm * TN + nn) v = acc[mm][nn];
    if (ctile < ntiles && row0 < p.M) tile_epilogue(p, row0, ctile, v, lane);
  }
}

// Row-major activation segments (the concatenated target layers) -> packed
// rows; rows from M up to the next multiple of 16 are zero.
template <typename T>
__global__ void pack_act_kernel(GemmArgs a, void* dst) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC, SZ = sizeof(T);
  const int nsteps = a.Kd / KC;
  const int mt = (a.M + 15) / 16;
  const int64_t total = (int64_t)mt * nsteps * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(q & 63);
    const int64_t ts = q >> 6;
    const int s = (int)(ts % nsteps), t = (int)(ts / nsteps);
    const int row = t * 16 + (l & 15);
    const int kk = s * KC + (l >> 4) * E;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < a.M) {
      const int seg = kk / a.a_seg_k, ks = kk % a.a_seg_k;
      v = load16(static_cast<const char*>(a.a_ptr[seg]) +
                 ((int64_t)row * a.lda + ks) * SZ);
    }
    *reinterpret_cast<u32x4*>(static_cast<char*>(dst) + q * 16) = v;
  }
}

// SK steps per LDS stage and PD stages in flight when the step count
// allows, else one step per stage and two in flight (steps are always even).
template <int TM, int TN, int WM, int WN, int SK, int PD>
hipError_t tiled_t(const GemmArgs& a, hipStream_t s) {
  using C = Tiled<TM, TN, WM, WN>;
  const int gm = (a.M + 16 * C::BMT - 1) / (16 * C::BMT);
  const int nbn = (a.N / 16 + C::BNT - 1) / C::BNT;
  const int grid = (nbn + 7) / 8 * 8 * gm;
  const int nsteps = a.Kd / Storage<bf16_t>::KC;
  if (nsteps % (SK * PD) == 0)
    launch_k((gemm_tiled_kernel<TM, TN, WM, WN, SK, PD>), dim3(grid),
                       dim3(64 * C::NW), 0, s, a, gm, nbn);
  else
    launch_k((gemm_tiled_kernel<TM, TN, WM, WN, 1, 2>), dim3(grid),
                       dim3(64 * C::NW), 0, s, a, gm, nbn);
  return hipGetLastError();
}

#ifndef DFLASH_T64_SK
#define DFLASH_T64_SK 2
#endif
#ifndef DFLASH_T64_PD
#define DFLASH_T64_PD 4
#endif
#ifndef DFLASH_T128_SK
#define DFLASH_T128_SK 2
#endif
#ifndef DFLASH_T128_PD
#define DFLASH_T128_PD 2
#endif
template <int TM, int TN, int WM, int WN, int NBUF>
hipError_t dma_t(const GemmArgs& a, hipStream_t s) {
  using C = Tiled<TM, TN, WM, WN>;
  const int gm = (a.M + 16 * C::BMT - 1) / (16 * C::BMT);
  const int nbn = (a.N / 16 + C::BNT - 1) / C::BNT;
  const int grid = (nbn + 7) / 8 * 8 * gm;
  launch_k((gemm_dma_kernel<TM, TN, WM, WN, NBUF>), dim3(grid),
           dim3(64 * C::NW), 0, s, a, gm, nbn);
  return hipGetLastError();
}

#ifndef DFLASH_TILED_DMA
#define DFLASH_TILED_DMA 1
#endif
#ifndef DFLASH_D64_NBUF
#define DFLASH_D64_NBUF 8
#endif
#ifndef DFLASH_D128_NBUF
#define DFLASH_D128_NBUF 4
#endif
hipError_t tiled_cfg(int cfg, const GemmArgs& a, hipStream_t s) {
  switch (cfg) {
    case TILE_64x64:
      if (DFLASH_TILED_DMA) return dma_t<1, 1, 2, 2, DFLASH_D64_NBUF>(a, s);
      return tiled_t<1, 1, 2, 2, DFLASH_T64_SK, DFLASH_T64_PD>(a, s);
    case TILE_128x128:
      if (DFLASH_TILED_DMA) return dma_t<2, 2, 2, 2, DFLASH_D128_NBUF>(a, s);
      return tiled_t<2, 2, 2, 2, DFLASH_T128_SK, DFLASH_T128_PD>(a, s);
    case TILE_256x64:
      if (DFLASH_TILED_DMA) return dma_t<4, 1, 2, 2, 4>(a, s);
      return tiled_t<4, 1, 2, 2, 2, 2>(a, s);
    case TILE_256x128:
      if (DFLASH_TILED_DMA) return dma_t<4, 2, 2, 2, 4>(a, s);
      return tiled_t<4, 2, 2, 2, 2, 1>(a, s);
    case TILE_128x256:
      if (DFLASH_TILED_DMA) return dma_t<2, 4, 2, 2, 4>(a, s);
      return tiled_t<2, 4, 2, 2, 2, 1>(a, s);
    case TILE_256x256:
      if (DFLASH_TILED_DMA) return dma_t<4, 2, 2, 4, 4>(a, s);
      return tiled_t<4, 2, 2, 4, 2, 2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

#ifndef DFLASH_TILED_CFG
#define DFLASH_TILED_CFG -1
#endif

// Block shape by rows and columns (measured on MI355X at 64, 256 and 1024
// rows over the drafter's projection and LM-head shapes).
int plan_tiled(int M, int N) {
  if (DFLASH_TILED_CFG >= 0) return DFLASH_TILED_CFG;
  if (M > 512) return TILE_128x128;
  if (M > 64 && N >= 16384) return TILE_128x128;
  return TILE_64x64;
}

hipError_t launch_gemm_tiled(bool bf16, int cfg, const GemmArgs& a,
                             hipStream_t s) {
  if (!bf16) return hipErrorInvalidValue;  // fp32 drafters use gemm_kernel
  return tiled_cfg(cfg, a, s);
}

hipError_t launch_pack_act(bool bf16, const GemmArgs& a, void* dst,
                           hipStream_t s) {
  const int KC = bf16 ? Storage<bf16_t>::KC : Storage<float>::KC;
  const int64_t chunks = (int64_t)((a.M + 15) / 16) * (a.Kd / KC) * 64;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    launch_k(pack_act_kernel<bf16_t>, dim3((unsigned)blocks),
                       dim3(256), 0, s, a, dst);
  else
    launch_k(pack_act_kernel<float>, dim3((unsigned)blocks),
                       dim3(256), 0, s, a, dst);
  return hipGetLastError();
}

}  // namespace dflash
