// MFMA GEMMs for the batched drafter: 64 to a few thousand rows, where the
// projections and the LM head are dense contractions rather than weight
// streams (bf16).
//
// A workgroup of WM x WN waves owns a (32 WM TM) x (32 WN TN) output block
// over the whole contraction; each wave owns TM x TN tiles of 32 x 32 and
// runs the 32x32x16 MFMA (on gfx950 it has twice the throughput of the
// 16x16x32 form).  Operands are packed fragment-major (1 KiB per 16 rows x
// one 32-wide contraction step), and each fragment goes from global memory
// straight into a ring of contraction steps in LDS (see gemm_dma_kernel).
// The projection epilogues run per wave on its own tiles straight from the
// accumulators (partner columns for RoPE and SwiGLU come from the lane 8
// apart); the LM head's top-2 reduction parks the block's logits in LDS and
// scans each row.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the mapping below
// gives the row blocks of one column block workgroup ids 8 apart, so they
// run on the same XCD and read that weight block through one L2.
#include "gemm_epilogue.h"

namespace dflash {

namespace {

template <int TM, int TN, int WM, int WN>
struct Tiled {
  static constexpr int NW = WM * WN;
  static constexpr int BMT = 2 * WM * TM;  // 16-row fragments per block
  static constexpr int BNT = 2 * WN * TN;  // 16-column fragments per block
  static constexpr int NF = BMT + BNT;     // fragments per contraction step
  static constexpr int LPW = NF / NW;      // fragment loads per wave per step
  static_assert(NF % NW == 0, "fragments must split evenly over the waves");
};

// Projection epilogue of one block of sums parked in LDS (L: BM rows of
// BN + 1 floats; block column c is column c % 16 of 16-column tile
// tile0 + c / 16).  Rows past M and tiles past N are skipped.
//   EP_STORE / EP_RESID: a unit is 4 consecutive columns of a row (float4
//   stores, 32 lanes along a row of 128 columns).
//   Pair epilogues: a unit is one (row, tile): its 8 low columns and their
//   partners, written as whole 16-byte chunks (pair_epilogue8); the lanes of
//   a wave take consecutive rows.
template <int BM, int BN, int NT>
__device__ __forceinline__ void block_epilogue(const GemmArgs& p,
                                               const float* L, int row0,
                                               int tile0) {
  const int ntiles = p.N / 16;
  if (p.ep == EP_STORE || p.ep == EP_RESID) {
    constexpr int UPR = BN / 4;
    for (int u = threadIdx.x; u < BM * UPR; u += NT) {
      const int r = u / UPR, c4 = (u % UPR) * 4;
      const int row = row0 + r, tile = tile0 + c4 / 16;
      if (row >= p.M || tile >= ntiles) continue;
      const float* lr = L + r * (BN + 1) + c4;
      if (p.cmap == MAP_LINEAR) {
        float* o = p.out_f32 + (int64_t)row * p.ldo + tile * 16 + c4 % 16;
        f32x4 v = {lr[0], lr[1], lr[2], lr[3]};
        if (p.ep == EP_RESID) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(o);
          v = f32x4{x[0] + v[0], x[1] + v[1], x[2] + v[2], x[3] + v[3]};
        }
        *reinterpret_cast<f32x4*>(o) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col =
              map_col(p.cmap, p.pair_group, p.pair_off, tile, c4 % 16 + e);
          float* o = p.out_f32 + (int64_t)row * p.ldo + col;
          *o = p.ep == EP_RESID ? *o + lr[e] : lr[e];
        }
      }
    }
    return;
  }
  constexpr int TPB = BN / 16;
  for (int u = threadIdx.x; u < BM * TPB; u += NT) {
    const int r = u % BM, tb = u / BM;
    const int row = row0 + r, tile = tile0 + tb;
    if (row >= p.M || tile >= ntiles) continue;
    const float* lr = L + r * (BN + 1) + tb * 16;
    float a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = lr[k];
      b[k] = lr[k + 8];
    }
    pair_epilogue8(p, row,
                   map_col(p.cmap, p.pair_group, p.pair_off, tile, 0), a, b);
  }
}

// LM-head reduction of one block of logits parked in LDS (L: BM rows of
// BN + 1 floats; the odd row stride makes a wave's column reads hit 64
// different banks).  NT threads, NT / BM per row: thread t scans row t % BM,
// its part t / BM of the columns, in increasing column order keeping (max,
// its lowest index, second max, sum of exp(z - max)); the parts are then
// merged in order and the row's record for this column block written:
// top2[row * nrec + rec].  Columns past N (the ragged last block) are
// skipped, rows past M are not written.
template <int BM, int BN, int NT>
__device__ __forceinline__ void top2_block(const GemmArgs& p, const float* L,
                                           Top2* part, int row0, int col0,
                                           int rec, int nrec) {
  static_assert(NT % BM == 0, "whole rows per thread group");
  constexpr int TPR = NT / BM, CPT = BN / TPR;
  const int t = threadIdx.x, r = t % BM, q = t / BM;
  const int row = row0 + r;
  const bool row_ok = row < p.M;
  float m1 = -INFINITY, m2 = -INFINITY, sum = 0.f;
  int i1 = 0x7fffffff;
  const float* lr = L + r * (BN + 1) + q * CPT;
  const int cbase = col0 + q * CPT;
#pragma unroll 8
  for (int i = 0; i < CPT; ++i) {
    const int col = cbase + i;
    if (col >= p.N) break;
    const float z = lr[i];
    if (z > m1) {
      sum = sum * __expf(m1 - z) + 1.f;
      m2 = m1;
      m1 = z;
      i1 = col;
    } else {
      m2 = fmaxf(m2, z);
      sum += __expf(z - m1);
    }
    if (p.logits != nullptr && row_ok) store_debug_logit(p, row, col, z);
  }
  Top2 v;
  v.m1 = m1;
  v.i1 = i1;
  v.m2 = m2;
  v.s = sum;
  part[t] = v;
  __syncthreads();
  if (q == 0 && row_ok) {
#pragma unroll
    for (int k = 1; k < TPR; ++k) v = top2_merge(v, part[t + k * BM]);
    p.top2[(int64_t)row * nrec + rec] = v;
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
//
// With ksplit > 1 the grid holds ksplit copies of the block grid; copy sp
// takes contraction steps [sp n / ksplit, (sp + 1) n / ksplit) and stores its
// fp32 block at out_f32 + sp M ldo (EP_STORE only; splitk_reduce_kernel sums
// the copies).
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs p,
                                                                int gm,
                                                                int nbn,
                                                                int ksplit) {
  using C = Tiled<TM, TN, WM, WN>;
  constexpr int STAGE = C::NF * 64;  // u32x4 per contraction step
  constexpr bool kHalfStep = TM * TN >= 8 || C::NW >= 16;
  // the ring, reused after the contraction for the block's sums
  constexpr int BM = 32 * WM * TM, BN = 32 * WN * TN;
  // A block whose sums and merge records do not fit in the 160 KiB of LDS
  // at once is parked and finished in two halves of rows (first the waves
  // of the lower half of wm).
  constexpr int HALVES =
      BM * (BN + 1) * 4 + 64 * C::NW * 16 > 160 * 1024 ? 2 : 1;
  constexpr int BMH = BM / HALVES;
  static_assert(WM % HALVES == 0, "whole waves per half");
  // (u32x4 units) parked sums, then the top-2 merge records of NT threads
  constexpr int RING = NBUF * STAGE;
  constexpr int LOGITS = (BMH * (BN + 1) + 3) / 4, PARTS = 64 * C::NW;
  constexpr int EPI = LOGITS + PARTS;
  __shared__ u32x4 lds[RING > EPI ? RING : EPI];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the block grid is a multiple of 8 ids, so b & 7 is still the XCD
  const int grid1 = (nbn + 7) / 8 * 8 * gm;
  const int sp = blockIdx.x / grid1, b = blockIdx.x % grid1;
  const int xcd = b & 7, k = b >> 3;
  const int mb = k % gm, nb = (k / gm) * 8 + xcd;
  if (nb >= nbn) return;  // whole workgroup: padding of the XCD mapping
  const int ksteps = p.Kd / Storage<bf16_t>::KC;
  const int s_begin = (int)((int64_t)sp * ksteps / ksplit);
  const int nsteps = (int)((int64_t)(sp + 1) * ksteps / ksplit) - s_begin;
  const int mtiles = (p.M + 15) / 16, ntiles = p.N / 16;
  const int wm = wave / WN, wn = wave % WN;
  if (ksplit > 1) p.out_f32 += (int64_t)sp * p.M * p.ldo;

  // fragment f = wave + i NW of a step
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
    src[i] = base + (((int64_t)t * ksteps + s_begin) * 64 + lane) * 16;
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
  vm_wait_n<(NBUF - 1) * C::LPW>();
  __syncthreads();
  if constexpr (!kHalfStep) {
    Ops r0, r1;
    read(r0, 0);
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
      iter(s, r0, r1);
      iter(s + 1, r1, r0);
    }
    if (s < nsteps) mul(r0);  // odd step count: the last step
  } else {
    // One half-step of operands in flight instead of a whole step (for
    // wide wave tiles or four waves per SIMD, where registers are short):
    // the second half of step s is read while the first is multiplied,
    // and the first half of step s + 1 while the second is.  Each
    // accumulator still sums the half-steps in order.
    using OpsH = u32x4[TM + TN];
    auto read_h = [&](OpsH& r, int slot, int h) {
      const u32x4* cur = lds + slot * STAGE;
#pragma unroll
      for (int m = 0; m < TM; ++m) r[m] = cur[a_off + m * 128 + 32 * h];
#pragma unroll
      for (int n = 0; n < TN; ++n) r[TM + n] = cur[w_off + n * 128 + 32 * h];
    };
    auto mul_h = [&](const OpsH& r) {
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) mma32(acc[m][n], r[m], r[TM + n]);
    };
    OpsH ra, rb;
    read_h(ra, 0, 0);
    for (int s = 0; s < nsteps; ++s) {
      read_h(rb, s % NBUF, 1);
      __builtin_amdgcn_sched_barrier(0);
      mul_h(ra);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < nsteps) {
        // this wave's loads of step s + 1 have landed; after the barrier
        // every wave's have, and every wave has read step s (the barrier
        // waits for this wave's LDS reads), so its slot can be refilled
        vm_wait_n<(NBUF - 2) * C::LPW>();
        __syncthreads();
        issue(s + NBUF, s % NBUF);
        read_h(ra, (s + 1) % NBUF, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      mul_h(rb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  vm_wait_n<0>();  // the clamped refills past the last step

  // FP8 weights: each column's sum times its row scale (one float rounding)
  float sc[TN];
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    const int col = nb * BN + (wn * TN + n) * 32 + (lane & 31);
    sc[n] = (p.wscale != nullptr && col < p.N) ? p.wscale[col] : 1.f;
  }
  float* L = reinterpret_cast<float*>(lds);  // [BMH][BN + 1]
#pragma unroll
  for (int h = 0; h < HALVES; ++h) {
    // Every wave has drained its loads and finished reading the ring (or
    // the previous half): park this half's sums there, then run the
    // epilogue over its whole rows.
    __syncthreads();
    if (wm / (WM / HALVES) == h) {
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = (wm * TM + m) * 32 + 4 * (lane >> 5) +
                          8 * (j >> 2) + (j & 3) - h * BMH;
            const int c = (wn * TN + n) * 32 + (lane & 31);
            L[r * (BN + 1) + c] =
                p.wscale != nullptr ? acc[m][n][j] * sc[n] : acc[m][n][j];
          }
    }
    __syncthreads();
    // (blocks parked in halves serve the LM head only: the projection
    // epilogues' registers on top of the live accumulators would spill)
    if (HALVES == 2 || p.ep == EP_TOP2)
      top2_block<BMH, BN, 64 * C::NW>(p, L,
                                      reinterpret_cast<Top2*>(lds + LOGITS),
                                      mb * BM + h * BMH, nb * BN, nb, nbn);
    else if constexpr (HALVES == 1)
      block_epilogue<BMH, BN, 64 * C::NW>(p, L, mb * BM + h * BMH,
                                          nb * C::BNT);
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

template <int TM, int TN, int WM, int WN, int NBUF>
hipError_t dma_t(const GemmArgs& a, int ksplit, hipStream_t s) {
  using C = Tiled<TM, TN, WM, WN>;
  const int gm = (a.M + 16 * C::BMT - 1) / (16 * C::BMT);
  const int nbn = (a.N / 16 + C::BNT - 1) / C::BNT;
  const int grid = (nbn + 7) / 8 * 8 * gm;
  launch_k((gemm_dma_kernel<TM, TN, WM, WN, NBUF>), dim3(grid * ksplit),
           dim3(64 * C::NW), 0, s, a, gm, nbn, ksplit);
  return hipGetLastError();
}

// out[row][col] (+)= sum over s of ws[s][row][col], s in order, fp32; one
// float4 per thread (N % 4 == 0).  S is a template argument so that the S
// copies (and the old output) are loaded together before the sum.
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    int M, int N, const float* ws, float* out, int ldo, int resid) {
  const int64_t n4 = (int64_t)M * N / 4, plane = (int64_t)M * N;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * 256) {
    const int64_t e = q * 4;
    const int row = (int)(e / N), col = (int)(e % N);
    float* o = out + (int64_t)row * ldo + col;
    f32x4 w[S], x{};
#pragma unroll
    for (int k = 0; k < S; ++k)
      w[k] = *reinterpret_cast<const f32x4*>(ws + k * plane + e);
    if (resid) x = *reinterpret_cast<const f32x4*>(o);
    f32x4 v = w[0];
#pragma unroll
    for (int k = 1; k < S; ++k)
      v = f32x4{v[0] + w[k][0], v[1] + w[k][1], v[2] + w[k][2], v[3] + w[k][3]};
    if (resid) v = f32x4{x[0] + v[0], x[1] + v[1], x[2] + v[2], x[3] + v[3]};
    *reinterpret_cast<f32x4*>(o) = v;
  }
}

// The pair epilogue (EP_QKV, EP_KV) of a split GEMM: its S copies were stored
// in tile order (tile t's 8 low columns, then their 8 partners, at columns
// 16t .. 16t + 15 of ws[s][row]).  One thread per (row, tile): the copies are
// added in order in float, then pair_epilogue8 finishes the 16 values as the
// unsplit kernel's epilogue does.
template <int S>
__global__ __launch_bounds__(256) void splitk_pair_kernel(GemmArgs p,
                                                          const float* ws) {
  const int ntiles = p.N / 16;
  const int64_t units = (int64_t)p.M * ntiles, plane = (int64_t)p.M * p.N;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * 256) {
    const int row = (int)(u / ntiles), tile = (int)(u % ntiles);
    const float* w = ws + (int64_t)row * p.N + tile * 16;
    f32x4 c[S][4];
#pragma unroll
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[k][j] = *reinterpret_cast<const f32x4*>(w + k * plane + 4 * j);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4 q = c[0][j];
#pragma unroll
      for (int k = 1; k < S; ++k)
        q = f32x4{q[0] + c[k][j][0], q[1] + c[k][j][1], q[2] + c[k][j][2],
                  q[3] + c[k][j][3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = q[e];
    }
    float a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[k] = v[k];
      b[k] = v[k + 8];
    }
    pair_epilogue8(p, row, map_col(p.cmap, p.pair_group, p.pair_off, tile, 0),
                   a, b);
  }
}

#ifndef DFLASH_D64_NBUF
#define DFLASH_D64_NBUF 8
#endif
#ifndef DFLASH_D128_NBUF
#define DFLASH_D128_NBUF 4
#endif
#ifndef DFLASH_D192_NBUF
#define DFLASH_D192_NBUF 4
#endif
#ifndef DFLASH_W8_NBUF
#define DFLASH_W8_NBUF 4
#endif
#ifndef DFLASH_W16_NBUF
#define DFLASH_W16_NBUF 4
#endif
hipError_t tiled_cfg(int cfg, const GemmArgs& a, int ks, hipStream_t s) {
  switch (cfg) {
    case TILE_64x64: return dma_t<1, 1, 2, 2, DFLASH_D64_NBUF>(a, ks, s);
    case TILE_128x128: return dma_t<2, 2, 2, 2, DFLASH_D128_NBUF>(a, ks, s);
    case TILE_256x64: return dma_t<4, 1, 2, 2, 4>(a, ks, s);
    case TILE_256x128: return dma_t<4, 2, 2, 2, 4>(a, ks, s);
    case TILE_128x256: return dma_t<2, 4, 2, 2, 4>(a, ks, s);
    case TILE_256x128_W8: return dma_t<2, 2, 4, 2, DFLASH_W8_NBUF>(a, ks, s);
    case TILE_128x192: return dma_t<2, 3, 2, 2, DFLASH_D192_NBUF>(a, ks, s);
    case TILE_128x128_W8: return dma_t<2, 1, 2, 4, DFLASH_D128_NBUF>(a, ks, s);
    case TILE_256x256:  // the LM head only
      if (a.ep != EP_TOP2) return hipErrorInvalidValue;
      return dma_t<2, 2, 4, 4, DFLASH_W16_NBUF>(a, ks, s);
  }
  return hipErrorInvalidValue;
}

// output columns per block of each shape
int tiled_block_cols(int cfg) {
  switch (cfg) {
    case TILE_64x64: case TILE_256x64: return 64;
    case TILE_128x128: case TILE_256x128: case TILE_256x128_W8:
    case TILE_128x128_W8:
      return 128;
    case TILE_128x256: case TILE_256x256: return 256;
    case TILE_128x192: return 192;
  }
  return 0;
}

}  // namespace

#ifndef DFLASH_TILED_CFG
#define DFLASH_TILED_CFG -1
#endif

#ifndef DFLASH_MID_ROWS
#define DFLASH_MID_ROWS 256
#endif
#ifndef DFLASH_O_UNSPLIT
#define DFLASH_O_UNSPLIT 1
#endif
#ifndef DFLASH_LM_W256_ROWS
#define DFLASH_LM_W256_ROWS 256
#endif

// Block shape by rows, columns and epilogue (measured on MI355X at 64, 256
// and 1024 rows over the drafter's projection and LM-head shapes).
int plan_tiled(int M, int N, int Kd, int ep, bool splittable) {
  if (DFLASH_TILED_CFG >= 0) return DFLASH_TILED_CFG;
  // 129 to 256 rows (measured at 240 and 256): the LM head takes one row
  // block of 256 x 128 on eight waves, so each weight block is read once
  // (240 x 151936: 346 against 369 us in 128 x 128), and a wide SwiGLU
  // output with a multiple of 192 columns takes 128 x 192 blocks, which
  // fill every CU where 128 x 128 gives half of them a second block
  // (256 x 24576: 69 against 84 us)
  if (M > 128 && M <= DFLASH_MID_ROWS) {
    if (ep == EP_TOP2) return TILE_256x128_W8;
    if (ep == EP_SWIGLU && N >= 16384 && N % 192 == 0) return TILE_128x192;
  }
  // beyond that the LM head takes 256 x 256 blocks on sixteen waves of
  // 64 x 64 (half the operand bytes per flop of 128 x 128, four waves per
  // SIMD; the logits parked and scanned in two halves): at 960 and 448 x
  // 151936 the batch-64 step 5.73-5.74 against 5.90-5.93 ms, where eight
  // waves of 128 x 64 gained nothing
  if (M > DFLASH_LM_W256_ROWS && ep == EP_TOP2) return TILE_256x256;
  // above 512 rows, outputs narrower than 16384 columns take 256 x 128
  // blocks on eight waves (with split-K filling the CUs): 16% faster than
  // 128 x 128 there at 1024 rows, slower for the wide gate/up and LM head.
  // Those that cannot split (QKV, the injected K/V) and have a multiple of
  // 192 columns take 128 x 192 blocks instead, which fill every CU where
  // 256 x 128 leaves a quarter idle (6144 columns at 1024 rows: 84 -> 74 us)
  if (M > 512 && N < 16384 && !splittable && N % 192 == 0)
    return TILE_128x192;
  // from 1024 rows a residual / store GEMM with a contraction of at most
  // 4096 (O) fills the grid in 128 x 128 blocks without a split (O at 1024
  // x 4096 x 4096 took 51 us against 41 us plus a 13 us reduction), and
  // above 512 rows so does a wide output (gate/up); both on eight waves of
  // 64 x 32, four waves per SIMD at two blocks per CU (O 47.3 against 52.4
  // us, gate/up 216.9 against 221.3 us on four waves of 64 x 64)
  if (M >= 1024 && N < 16384 && splittable && Kd <= 4096 &&
      DFLASH_O_UNSPLIT)
    return TILE_128x128_W8;
  if (M > 512) return N >= 16384 ? TILE_128x128_W8 : TILE_256x128_W8;
  // from 65 rows: 128 x 128 for wide outputs, and for narrow ones whose
  // contraction can be split over the grid (at 256 rows the residual and
  // store GEMMs take 30 us plus the reduction, against 44 us in 64 x 64)
  if (M > 64 && (N >= 16384 || splittable)) return TILE_128x128;
  return TILE_64x64;
}

int tiled_top2_records(int cfg, int N) {
  const int bc = tiled_block_cols(cfg);
  return bc > 0 ? (N + bc - 1) / bc : 0;
}

int tiled_blocks(int cfg, int M, int N) {
  const int bc = tiled_block_cols(cfg);
  const int br = cfg == TILE_64x64 ? 64
                 : (cfg == TILE_128x128 || cfg == TILE_128x256 ||
                    cfg == TILE_128x192 || cfg == TILE_128x128_W8)
                     ? 128
                     : 256;
  return bc > 0 ? ((M + br - 1) / br) * ((N + bc - 1) / bc) : 0;
}

hipError_t launch_gemm_tiled(bool bf16, int cfg, const GemmArgs& a,
                             int ksplit, hipStream_t s) {
  // fp32 drafters use gemm_kernel; FP8 weights come here widened to bf16
  if (!bf16 || a.wfp8) return hipErrorInvalidValue;
  // every split needs at least one contraction step
  if (ksplit < 1 || ksplit > a.Kd / Storage<bf16_t>::KC ||
      (ksplit > 1 && a.ep != EP_STORE))
    return hipErrorInvalidValue;
  return tiled_cfg(cfg, a, ksplit, s);
}

hipError_t launch_splitk_reduce(int M, int N, int S, const float* ws,
                                float* out, int ldo, bool resid,
                                hipStream_t s) {
  if (N % 4 != 0 || ldo % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)M * N / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks);
  const int r = resid ? 1 : 0;
  switch (S) {  // 1 to 4 copies (the most a split GEMM makes)
    case 1: launch_k(splitk_reduce_kernel<1>, grid, dim3(256), 0, s, M, N, ws, out, ldo, r); break;
    case 2: launch_k(splitk_reduce_kernel<2>, grid, dim3(256), 0, s, M, N, ws, out, ldo, r); break;
    case 3: launch_k(splitk_reduce_kernel<3>, grid, dim3(256), 0, s, M, N, ws, out, ldo, r); break;
    case 4: launch_k(splitk_reduce_kernel<4>, grid, dim3(256), 0, s, M, N, ws, out, ldo, r); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_pair(const GemmArgs& a, int S, const float* ws,
                              hipStream_t s) {
  if (a.cmap != MAP_PAIRS || (a.ep != EP_QKV && a.ep != EP_KV) ||
      a.N % 16 != 0)
    return hipErrorInvalidValue;
  const int64_t units = (int64_t)a.M * (a.N / 16);
  int64_t blocks = (units + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks);
  switch (S) {  // 2 to 4 copies (the most a split GEMM makes)
    case 2: launch_k(splitk_pair_kernel<2>, grid, dim3(256), 0, s, a, ws); break;
    case 3: launch_k(splitk_pair_kernel<3>, grid, dim3(256), 0, s, a, ws); break;
    case 4: launch_k(splitk_pair_kernel<4>, grid, dim3(256), 0, s, a, ws); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
