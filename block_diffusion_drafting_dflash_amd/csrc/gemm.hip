// MFMA GEMMs of the drafter (projections and LM head) on packed operands.
//
// At batch 1 the job is streaming each weight byte from HBM exactly once.
// Weights are packed once into fragment-major order (see kernels.h), so each
// wave-wide weight load is one contiguous 1 KiB burst; the activation rows are
// written packed by the kernels that produce them, so their loads are
// contiguous too.  A workgroup owns one 16-column output tile over the whole
// contraction: its waves take interleaved fragment steps, keep several steps
// of loads in flight, and sum their tiles through LDS in wave order.  The
// finished tile is handled by the same workgroup (residual add, RoPE and the
// KV-cache scatter, SwiGLU, the LM-head top-2 reduction), so no workgroup
// ever waits on another.
#include "gemm_epilogue.h"

namespace dflash {

namespace {

// Waves per workgroup and fragment steps in flight per wave at batch 1
// (one 16-row tile); measured on MI355X.
#ifndef DFLASH_GEMM_W
#define DFLASH_GEMM_W 8
#endif
#ifndef DFLASH_GEMM_U
#define DFLASH_GEMM_U 4
#endif
#ifndef DFLASH_LM_W
#define DFLASH_LM_W 16
#endif
#ifndef DFLASH_LM_U
#define DFLASH_LM_U 8
#endif
// Persistent LM head (batches of up to 16 rows): waves per workgroup and the
// most contraction steps a wave holds (bf16 hidden <= 16 * 8 * 32, fp32
// hidden <= 16 * 8 * 16).
#ifndef DFLASH_LMP_W
#define DFLASH_LMP_W 16
#endif
#ifndef DFLASH_LMP_NS
#define DFLASH_LMP_NS 8
#endif
// An FP8 gate/up projection of up to 16 rows takes the persistent stream
// when it has at least this many 16-column tiles per compute unit: the
// activation fragments, twice the bytes of the FP8 weight fragments they
// meet, are then loaded once per workgroup instead of once per tile.
// Measured at the Qwen3-8B shape (4096 x 24576, six tiles per workgroup):
// the FP8 step 2.2 us faster; with bf16 weights the stream was 3 us slower
// than the per-tile workgroups, so bf16 keeps those.
#ifndef DFLASH_PROJ_STREAM_MIN
#define DFLASH_PROJ_STREAM_MIN 2
#endif


// acc[m] over this wave's share of the contraction.  With F64 each MFMA
// step (32 contraction elements) is summed in fp32 from zero and added to a
// float64 accumulator: the projections feed bf16-rounded activations of the
// next step, where fp32 accumulation error over thousands of terms flips
// roundings that then spread through the layer.  The LM head's logits feed
// nothing further and accumulate in fp32.
// The same over FP8 step-pair weights (packed A): a wave takes pairs wave,
// wave + W, ...; each pair's weight load is widened to two bf16 fragments.
template <int MT, int W, int U, bool F64>
__device__ __forceinline__ void gemm_core_fp8(const GemmArgs& p, int tile,
                                              int m_base,
                                              double (&acc)[MT][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int npairs = p.Kd / 64, nsteps = p.Kd / 32;
  const char* wbase =
      static_cast<const char*>(p.w) + ((int64_t)tile * npairs * 64 + lane) * 16;
  const char* abase[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mt = min(m_base / 16 + m, (p.M + 15) / 16 - 1);
    abase[m] = static_cast<const char*>(p.a_ptr[0]) +
               ((int64_t)mt * nsteps * 64 + lane) * 16;
  }
  f32x4 acc32[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc32[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = 0.0;
  }
  auto step = [&](int m, u32x4 a, u32x4 b) {
    if constexpr (F64) {
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      mma16(t, a, b, bf16_t());
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] += (double)t[j];
    } else {
      mma16(acc32[m], a, b, bf16_t());
    }
  };
  int s = wave;
  for (; s + (U - 1) * W < npairs; s += U * W) {
    u32x4 bw[U], af[U][MT][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
      bw[u] = load16(wbase + (int64_t)(s + u * W) * 1024);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        af[u][m][0] = load16(abase[m] + (int64_t)(2 * (s + u * W)) * 1024);
        af[u][m][1] = load16(abase[m] + (int64_t)(2 * (s + u * W) + 1) * 1024);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 b0 = fp8x8_to_bf16(bw[u].x, bw[u].y);
      const u32x4 b1 = fp8x8_to_bf16(bw[u].z, bw[u].w);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        step(m, af[u][m][0], b0);
        step(m, af[u][m][1], b1);
      }
    }
  }
  for (; s < npairs; s += W) {
    const u32x4 bw = load16(wbase + (int64_t)s * 1024);
    const u32x4 b0 = fp8x8_to_bf16(bw.x, bw.y);
    const u32x4 b1 = fp8x8_to_bf16(bw.z, bw.w);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      step(m, load16(abase[m] + (int64_t)(2 * s) * 1024), b0);
      step(m, load16(abase[m] + (int64_t)(2 * s + 1) * 1024), b1);
    }
  }
  if constexpr (!F64) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] += (double)acc32[m][j];
  }
}

template <typename T, int MT, int AP, int W, int U, bool F64>
__device__ __forceinline__ void gemm_core(const GemmArgs& p, int tile,
                                          int m_base, double (&acc)[MT][4]) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC, SZ = sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = p.Kd / KC;
  const char* wbase =
      static_cast<const char*>(p.w) + ((int64_t)tile * nsteps * 64 + lane) * 16;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = 0.0;
  auto fold = [&](int m, const f32x4& t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] += (double)t[j];
  };
  f32x4 acc32[MT];  // without F64: fp32 across all steps
#pragma unroll
  for (int m = 0; m < MT; ++m) acc32[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A operand addressing: packed fragments, or row-major segments
  const int sps = AP ? nsteps : p.a_seg_k / KC;  // steps per segment
  const int nseg = AP ? 1 : (nsteps + sps - 1) / sps;
  int64_t aoff[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (AP) {
      const int mt = min(m_base / 16 + m, (p.M + 15) / 16 - 1);
      aoff[m] = ((int64_t)mt * nsteps * 64 + lane) * 16;
    } else {
      const int row = min(m_base + 16 * m + r, p.M - 1);
      aoff[m] = ((int64_t)row * p.lda + g * E) * SZ;
    }
  }
  for (int seg = 0; seg < nseg; ++seg) {
    const int s0 = seg * sps, s1 = min(nsteps, s0 + sps);
    const char* abase = static_cast<const char*>(p.a_ptr[seg]);
    // A fragment of step s within this segment
    auto a_at = [&](int m, int s) -> const char* {
      return AP ? abase + aoff[m] + (int64_t)s * 1024
                : abase + aoff[m] + (int64_t)(s - s0) * KC * SZ;
    };
    int s = s0 + ((wave - s0) % W + W) % W;
    for (; s + (U - 1) * W < s1; s += U * W) {
      u32x4 bf[U], af[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u)
        bf[u] = load16(wbase + (int64_t)(s + u * W) * 1024);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) af[u][m] = load16(a_at(m, s + u * W));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if constexpr (F64) {
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            mma16(t, af[u][m], bf[u], T());
            fold(m, t);
          } else {
            mma16(acc32[m], af[u][m], bf[u], T());
          }
        }
    }
    for (; s < s1; s += W) {
      const u32x4 bf = load16(wbase + (int64_t)s * 1024);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if constexpr (F64) {
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
          mma16(t, load16(a_at(m, s)), bf, T());
          fold(m, t);
        } else {
          mma16(acc32[m], load16(a_at(m, s)), bf, T());
        }
      }
    }
  }
  if constexpr (!F64) {
#pragma unroll
    for (int m = 0; m < MT; ++m) fold(m, acc32[m]);
  }
}

// Packed A operand, software-pipelined: a wave takes the steps wave,
// wave + W, ... of the contraction in blocks of U, and two register sets
// alternate, so that while one block is multiplied the loads of the next
// are in flight.  The loads are the staging loads with exact waits: the
// compiler's own waits would drain both sets at every loop edge.
// With WF8 a unit is a pair of contraction steps: one FP8 weight load (two
// steps) and two A fragments per row tile; otherwise one step.
template <int AHEAD, int NL, int U, int MT, typename T, bool F64, bool WF8>
__device__ __forceinline__ void packed_block(u32x4 (&st)[NL], int first,
                                             int n_i, double (&acc)[MT][4],
                                             f32x4 (&acc32)[MT]) {
  constexpr int AS = WF8 ? 2 : 1, UL = 1 + AS * MT;
  stage_wait<0, NL, AHEAD>(st);
  auto step = [&](int m, u32x4 a, u32x4 b) {
    if constexpr (F64) {
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      mma16(t, a, b, T());
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] += (double)t[j];
    } else {
      mma16(acc32[m], a, b, T());
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (first + u >= n_i) break;  // uniform: past this wave's last step
    if constexpr (WF8) {
      const u32x4 w = st[u * UL];
      const u32x4 b0 = fp8x8_to_bf16(w.x, w.y), b1 = fp8x8_to_bf16(w.z, w.w);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        step(m, st[u * UL + 1 + 2 * m], b0);
        step(m, st[u * UL + 2 + 2 * m], b1);
      }
    } else {
#pragma unroll
      for (int m = 0; m < MT; ++m) step(m, st[u * UL + 1 + m], st[u * UL]);
    }
  }
}

template <typename T, int MT, int W, int U, bool F64, bool WF8>
__device__ __forceinline__ void gemm_core_packed(const GemmArgs& p, int tile,
                                                 int m_base,
                                                 double (&acc)[MT][4]) {
  constexpr int KC = Storage<T>::KC;
  constexpr int AS = WF8 ? 2 : 1;
  constexpr int UL = 1 + AS * MT;  // loads per unit: weight, then A tiles
  constexpr int NL = U * UL;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = p.Kd / KC;
  const int nunits = WF8 ? nsteps / 2 : nsteps;
  const char* wbase =
      static_cast<const char*>(p.w) + ((int64_t)tile * nunits * 64 + lane) * 16;
  const char* abase[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int mt = min(m_base / 16 + m, (p.M + 15) / 16 - 1);
    abase[m] = static_cast<const char*>(p.a_ptr[0]) +
               ((int64_t)mt * nsteps * 64 + lane) * 16;
  }
  f32x4 acc32[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    acc32[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = 0.0;
  }
  const int n_i = wave < nunits ? (nunits - 1 - wave) / W + 1 : 0;
  const int nb = (n_i + U - 1) / U;
  // block b holds this wave's units bU .. bU + U - 1 (clamped to the last)
  auto load = [&](u32x4(&st)[NL], int blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(blk * U + u, n_i - 1);
      const int unit = wave + i * W;
      st[u * UL] = stage_load(wbase + (int64_t)unit * 1024);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int h = 0; h < AS; ++h)
          st[u * UL + 1 + AS * m + h] =
              stage_load(abase[m] + (int64_t)(AS * unit + h) * 1024);
    }
  };
  if (nb > 0) {
    // Straight-line shape: both sets loaded, pairs of blocks while a refill
    // exists, then the last pair with no refill.  Every set has a single
    // consumer, so no in-flight register is ever copied.  With an odd block
    // count the last refill of s1 (or, for one block, s1 itself) repeats
    // the wave's last unit and is not multiplied.
    u32x4 s0[NL], s1[NL];
    load(s0, 0);
    load(s1, 1);
    int blk = 0;
    for (; blk + 2 < nb; blk += 2) {
      packed_block<NL, NL, U, MT, T, F64, WF8>(s0, blk * U, n_i, acc, acc32);
      load(s0, blk + 2);
      packed_block<NL, NL, U, MT, T, F64, WF8>(s1, (blk + 1) * U, n_i, acc,
                                               acc32);
      load(s1, blk + 3);
    }
    packed_block<NL, NL, U, MT, T, F64, WF8>(s0, blk * U, n_i, acc, acc32);
    packed_block<0, NL, U, MT, T, F64, WF8>(s1, (blk + 1) * U, n_i, acc, acc32);
  }
  if constexpr (!F64) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] += (double)acc32[m][j];
  }
}

// Sums the waves' tiles in wave order (float64, one row tile at a time
// through redd); red[(m*4 + j)*64 + lane] then holds row 16m + 4(lane/16) + j,
// tile column lane % 16.
// With FP8 weights each column's sum is multiplied by its row scale before
// the one rounding to float.
template <int MT, int W>
__device__ __forceinline__ void reduce_waves(const double (&acc)[MT][4],
                                             double* redd, float* red,
                                             const float* wscale, int tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) redd[wave * 256 + j * 64 + lane] = acc[m][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < 256; idx += W * 64) {
      double v = redd[idx];
#pragma unroll
      for (int w = 1; w < W; ++w) v += redd[w * 256 + idx];
      if (wscale != nullptr) v *= (double)wscale[tile * 16 + (idx & 15)];
      red[m * 256 + idx] = (float)v;
    }
    __syncthreads();
  }
}

template <typename T, int MT, int W>
__device__ void apply_epilogue(const GemmArgs& p, int tile, int m_base,
                               const float* red) {
  constexpr int S = MT * 256;
  const int tid = threadIdx.x;
  auto row_of = [&](int idx) {
    return m_base + 16 * (idx >> 8) + 4 * ((idx & 63) >> 4) + ((idx >> 6) & 3);
  };
  if (p.ep == EP_STORE || p.ep == EP_RESID) {
    for (int idx = tid; idx < S; idx += W * 64) {
      const int row = row_of(idx);
      if (row >= p.M) continue;
      const int col = map_col(p.cmap, p.pair_group, p.pair_off, tile, idx & 15);
      float* o = p.out_f32 + (int64_t)row * p.ldo + col;
      *o = p.ep == EP_RESID ? *o + red[idx] : red[idx];
    }
    return;
  }
  if (p.ep == EP_TOP2) {
    // one thread per (row, column); the 16 columns of a row are 16
    // consecutive lanes of one wave
    for (int base = 0; base < S; base += W * 64) {
      const int idx = base + tid;
      const int row = row_of(idx);
      const int col = tile * 16 + (idx & 15);
      Top2 v = top2_empty();
      if (idx < S && row < p.M && col < p.N) {
        const float z = red[idx];
        v.m1 = z;
        v.i1 = col;
        v.s = 1.f;
        if (p.logits != nullptr) store_debug_logit(p, row, col, z);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) v = top2_merge(v, top2_shfl_xor(v, o));
      if (idx < S && (idx & 15) == 0 && row < p.M)
        p.top2[(int64_t)row * (p.N / 16) + tile] = v;
    }
    return;
  }
  // pair epilogues: tile column c < 8 with its partner c + 8
  for (int q = tid; q < MT * 128; q += W * 64) {
    const int c = q & 7, rg = (q >> 3) & 3, j = (q >> 5) & 3, m = q >> 7;
    const int idx = (m * 4 + j) * 64 + rg * 16 + c;
    const int row = m_base + 16 * m + 4 * rg + j;
    if (row >= p.M) continue;
    const int col = map_col(p.cmap, p.pair_group, p.pair_off, tile, c);
    pair_epilogue<T>(p, row, col, red[idx], red[idx + 8]);
  }
}

// PIPE: the software-pipelined core (packed A only; it holds two blocks of
// U steps in registers, so it suits workgroups of up to 8 waves)
// WF8: FP8 step-pair weights (bf16 drafters, packed A).
template <typename T, int MT, int AP, int W, int U, bool F64, bool PIPE,
          bool WF8>
__global__ __launch_bounds__(64 * W) void gemm_kernel(GemmArgs p) {
  static_assert(!PIPE || AP, "the pipelined core reads packed A");
  static_assert(!WF8 || AP, "FP8 weights take packed A");
  __shared__ double redd[W * 256];
  __shared__ float red[MT * 256];
  const int tile = blockIdx.x, m_base = blockIdx.y * 16 * MT;
  double acc[MT][4];
  if constexpr (PIPE)
    gemm_core_packed<T, MT, W, U, F64, WF8>(p, tile, m_base, acc);
  else if constexpr (WF8)
    gemm_core_fp8<MT, W, U, F64>(p, tile, m_base, acc);
  else
    gemm_core<T, MT, AP, W, U, F64>(p, tile, m_base, acc);
  reduce_waves<MT, W>(acc, redd, red, p.wscale, tile);
  apply_epilogue<T, MT, W>(p, tile, m_base, red);
}

// A SwiGLU pair whose bf16 rounding the float evaluation leaves open.
struct SlowPair {
  float a, b;
  int row, col;
};
// Tiles per workgroup of the persistent gate/up projection: each tile queues
// at most 16 x 8 pairs.
constexpr int kProjMaxTiles = 16;
constexpr int kSlowCap = kProjMaxTiles * 128;

// LM head for up to 16 drafted rows: one persistent workgroup per compute
// unit streams every P-th 16-column vocabulary tile (the workgroups sweep
// the matrix together).  With PROJ the same sweep serves the FP8 gate/up
// projection (EP_SWIGLU, contraction up to 16 W NS steps): each MFMA step is
// summed in fp32 from zero and added to a float64 accumulator, as in
// gemm_kernel, and each tile's pairs go through SwiGLU instead of the top-2
// reduction.  Only that epilogue is built in, and only its float evaluation
// runs between tiles: the pairs it leaves open are queued in LDS and take the
// float64 evaluation after the last tile, so the loop holds no float64
// exponential (its constants would crowd the registers and its spill reloads
// would wait for the loads in flight).
// Each wave keeps its share of the activation fragments in registers for
// the workgroup's lifetime, and the weight fragments of the next two tiles
// are in flight in two register sets while the current tile is multiplied,
// summed over the waves and reduced to top-2 records, so the weight stream
// does not pause at tile boundaries.  An LM-head tile is summed exactly as
// in gemm_kernel (fp32 over a wave's steps, then float64 over the waves in
// wave order); each row's record is merged over the workgroup's tiles in
// tile order and written once per workgroup: part[row][workgroup].

// AHEAD: staging loads issued after this tile's set (the other set's, or
// none for the last tile).  The tile is multiplied from set b; with REFILL
// b is then reloaded with the tile two ahead, before the wave sums.  With
// WF8 each of the NB weight loads of a set is a pair of contraction steps
// (activation fragments a[2u], a[2u + 1]); otherwise one step (a[u]).  The
// tile's 16 row scales (WF8) are scalar loads through the constant address
// space: a vector load here would make its use wait for every load in
// flight, the next tiles' weights included.
template <typename T, int W, int NA, int NB, int AHEAD, bool REFILL, bool WF8,
          bool PROJ, typename LoadW>
__device__ __forceinline__ void lm_tile(const GemmArgs& p, u32x4 (&a)[NA],
                                        u32x4 (&b)[NB], int n_i, int i,
                                        int tile, bool valid, double* redd,
                                        Top2& run, SlowPair* slow,
                                        int* slow_n, const LoadW& load_w) {
  float s16[16];
  if constexpr (WF8) {
    typedef const float __attribute__((address_space(4))) cfloat;
    const uint64_t ad = (uint64_t)(uintptr_t)(p.wscale + (int64_t)tile * 16);
    const uint64_t au =
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ad);
    const cfloat* ws = (const cfloat*)(uintptr_t)au;
#pragma unroll
    for (int c = 0; c < 16; ++c) s16[c] = ws[c];
  }
  stage_wait<0, NB, AHEAD>(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  double acc64[4] = {0.0, 0.0, 0.0, 0.0};
  auto step = [&](u32x4 x, u32x4 w) {
    if constexpr (PROJ) {
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
      mma16(t, x, w, T());
#pragma unroll
      for (int j = 0; j < 4; ++j) acc64[j] += (double)t[j];
    } else {
      mma16(acc, x, w, T());
    }
  };
#pragma unroll
  for (int s = 0; s < NB; ++s)
    if (s < n_i) {
      if constexpr (WF8) {
        step(a[2 * s], fp8x8_to_bf16(b[s].x, b[s].y));
        step(a[2 * s + 1], fp8x8_to_bf16(b[s].z, b[s].w));
      } else {
        step(a[s], b[s]);
      }
    }
  if constexpr (REFILL) load_w(b, i + 2);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    redd[wave * 256 + j * 64 + lane] = PROJ ? acc64[j] : (double)acc[j];
  __syncthreads();
  if (threadIdx.x < 256 && valid) {
    const int idx = threadIdx.x;
    // idx = (j, row group, column): row 4 (idx % 64 / 16) + idx / 64
    double v = redd[idx];
#pragma unroll
    for (int w = 1; w < W; ++w) v += redd[w * 256 + idx];
    if constexpr (WF8) {
      float sc = s16[0];
#pragma unroll
      for (int c = 1; c < 16; ++c) sc = (idx & 15) == c ? s16[c] : sc;
      v *= (double)sc;
    }
    const float z = (float)v;
    const int row = 4 * ((idx & 63) >> 4) + (idx >> 6);
    if constexpr (PROJ) {
      // tile column c < 8 pairs with c + 8, eight lanes up in the same wave
      const float zb = __shfl_down(z, 8, 16);
      const int c = idx & 15;
      if (c < 8 && row < p.M) {
        const int col = map_col(p.cmap, p.pair_group, p.pair_off, tile, c);
        uint32_t bits;
        if (swiglu_bf16_float(z, zb, bits)) {
          static_cast<bf16_t*>(p.out_t)
              [packed_offset<bf16_t>(row, col, p.pair_off) / 2]
                  .bits = (uint16_t)bits;
        } else {
          // < kSlowCap: the host bounds the tiles per workgroup
          const int q = atomicAdd(slow_n, 1);
          if (q < kSlowCap) slow[q] = SlowPair{z, zb, row, col};
        }
      }
      return;
    }
    const int col = tile * 16 + (idx & 15);
    Top2 t = top2_empty();
    if (row < p.M) {
      t.m1 = z;
      t.i1 = col;
      t.s = 1.f;
      if (p.logits != nullptr) store_debug_logit(p, row, col, z);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) t = top2_merge(t, top2_shfl_xor(t, o));
    run = top2_merge(run, t);
  }
}

// NS: the most contraction steps a wave holds.  A wave's units (steps, or
// with WF8 pairs of steps) are wave, wave + W, ...
template <typename T, int W, int NS, bool WF8, bool PROJ>
__device__ __forceinline__ void persistent_sweep(const GemmArgs& p) {
  static_assert(!PROJ || WF8, "the SwiGLU stream takes FP8 weights");
  constexpr int KC = Storage<T>::KC;
  constexpr int NB = WF8 ? NS / 2 : NS;  // weight loads per tile per wave
  __shared__ double redd[2][W * 256];
  __shared__ SlowPair slow[PROJ ? kSlowCap : 1];
  __shared__ int slow_n;
  if (threadIdx.x == 0) slow_n = 0;  // first used after a barrier
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = p.Kd / KC;
  const int nunits = WF8 ? nsteps / 2 : nsteps;
  const int ntiles = p.N / 16, P = gridDim.x, wg = blockIdx.x;
  // tiles wg, wg + P, ...: the workgroups sweep the matrix together
  const int nt = (ntiles - 1 - wg) / P + 1;  // >= 1: P <= ntiles
  auto tile_of = [&](int i) { return wg + min(i, nt - 1) * P; };
  // this wave's units: wave, wave + W, ... (n_i of them, n_i <= NB)
  const int n_i = wave < nunits ? (nunits - 1 - wave) / W + 1 : 0;
  const int first = n_i > 0 ? wave : 0;  // a wave with no units reads unit 0
  const int64_t unit_off = (int64_t)first * 1024 + lane * 16;
  // a unit past the wave's last repeats the last, a slot past the last tile
  // repeats the last tile; neither is multiplied or summed
  auto load_w = [&](u32x4(&b)[NB], int i) {  // this workgroup's i-th tile
    const char* wt = static_cast<const char*>(p.w) +
                     (int64_t)tile_of(i) * nunits * 1024 + unit_off;
#pragma unroll
    for (int s = 0; s < NB; ++s)
      b[s] = stage_load(wt + (int64_t)min(s, max(n_i - 1, 0)) * W * 1024);
  };
  u32x4 a[NS], b0[NB], b1[NB];
  {
    const char* at = static_cast<const char*>(p.a_ptr[0]) + lane * 16;
#pragma unroll
    for (int s = 0; s < NB; ++s) {
      const int64_t unit = first + (int64_t)min(s, max(n_i - 1, 0)) * W;
      if constexpr (WF8) {
        a[2 * s] = stage_load(at + (2 * unit) * 1024);
        a[2 * s + 1] = stage_load(at + (2 * unit + 1) * 1024);
      } else {
        a[s] = stage_load(at + unit * 1024);
      }
    }
  }
  load_w(b0, 0);
  load_w(b1, 1);
  stage_wait<0, NS, 2 * NB>(a);
  Top2 run = top2_empty();
  int i = 0;
  for (; i + 2 < nt; i += 2) {
    lm_tile<T, W, NS, NB, NB, true, WF8, PROJ>(p, a, b0, n_i, i, tile_of(i),
                                               true, redd[0], run, slow,
                                               &slow_n, load_w);
    lm_tile<T, W, NS, NB, NB, true, WF8, PROJ>(p, a, b1, n_i, i + 1,
                                               tile_of(i + 1), true, redd[1],
                                               run, slow, &slow_n, load_w);
  }
  lm_tile<T, W, NS, NB, NB, false, WF8, PROJ>(p, a, b0, n_i, i, tile_of(i),
                                              true, redd[0], run, slow,
                                              &slow_n, load_w);
  // the second set was loaded whether or not its tile exists: wait for it
  // either way (only its sums are skipped)
  lm_tile<T, W, NS, NB, 0, false, WF8, PROJ>(p, a, b1, n_i, i + 1,
                                             tile_of(i + 1), i + 1 < nt,
                                             redd[1], run, slow, &slow_n,
                                             load_w);
  if constexpr (PROJ) {
    // nothing is in flight now: the queued pairs' float64 evaluation
    __syncthreads();
    const int n = min(slow_n, kSlowCap);
    for (int q = threadIdx.x; q < n; q += 64 * W) {
      const SlowPair e = slow[q];
      static_cast<bf16_t*>(p.out_t)
          [packed_offset<bf16_t>(e.row, e.col, p.pair_off) / 2]
              .bits = (uint16_t)swiglu_bf16_f64(e.a, e.b);
    }
    return;
  }
  if (threadIdx.x < 256 && (threadIdx.x & 15) == 0) {
    const int row = 4 * ((threadIdx.x & 63) >> 4) + (threadIdx.x >> 6);
    if (row < p.M) p.top2[(int64_t)row * P + wg] = run;
  }
}

template <typename T, int W, int NS, bool WF8>
__global__ __launch_bounds__(64 * W) void lm_head_kernel(GemmArgs p) {
  persistent_sweep<T, W, NS, WF8, false>(p);
}

// The FP8 gate/up projection on the same sweep (its own name in traces).
template <int W, int NS>
__global__ __launch_bounds__(64 * W) void gemm_stream_kernel(GemmArgs p) {
  persistent_sweep<bf16_t, W, NS, true, true>(p);
}

// One 16-byte chunk of the packed matrix per thread.
template <typename T>
__global__ void pack_kernel(PackArgs a) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC;
  const int nsteps = a.K / KC;
  const int64_t total = (int64_t)a.N / 16 * nsteps * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(q & 63);
    const int64_t ts = q >> 6;
    const int s = (int)(ts % nsteps), t = (int)(ts / nsteps);
    const int row = map_col(a.cmap, a.pair_group, a.pair_off, t, l & 15);
    int sg = 0;
    while (sg + 1 < a.nseg && row >= a.n0[sg + 1]) ++sg;
    const char* src = static_cast<const char*>(a.src[sg]) +
                      ((int64_t)(row - a.n0[sg]) * a.K + s * KC + (l >> 4) * E) *
                          (int64_t)sizeof(T);
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.dst) + q * 16) = load16(src);
  }
}

// FP8 E4M3 codes [N][K] (1 byte each): PACK_FP8 writes the step-pair layout
// (one 16-byte chunk per thread: 8 codes of each step of a pair);
// PACK_FP8_BF16 writes the bf16 layout with every code widened exactly.
__global__ void pack_fp8_kernel(PackArgs a) {
  const bool pairs = a.mode == PACK_FP8;
  const int units = pairs ? a.K / 64 : a.K / 32;
  const int64_t total = (int64_t)a.N / 16 * units * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(q & 63);
    const int64_t ts = q >> 6;
    const int s = (int)(ts % units), t = (int)(ts / units);
    const int row = map_col(a.cmap, a.pair_group, a.pair_off, t, l & 15);
    int sg = 0;
    while (sg + 1 < a.nseg && row >= a.n0[sg + 1]) ++sg;
    const unsigned char* src = static_cast<const unsigned char*>(a.src[sg]) +
                               (int64_t)(row - a.n0[sg]) * a.K;
    u32x4 v;
    if (pairs) {
      const u32x2 lo = *reinterpret_cast<const u32x2*>(src + s * 64 + (l >> 4) * 8);
      const u32x2 hi =
          *reinterpret_cast<const u32x2*>(src + s * 64 + 32 + (l >> 4) * 8);
      v = u32x4{lo.x, lo.y, hi.x, hi.y};
    } else {
      const u32x2 c = *reinterpret_cast<const u32x2*>(src + s * 32 + (l >> 4) * 8);
      v = fp8x8_to_bf16(c.x, c.y);
    }
    *reinterpret_cast<u32x4*>(static_cast<char*>(a.dst) + q * 16) = v;
  }
}

// Per-row scales (float) into packed column order: dst[16 t + c].
__global__ void pack_scale_kernel(PackArgs a) {
  const int n = a.N;
  for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += gridDim.x * blockDim.x) {
    const int row = map_col(a.cmap, a.pair_group, a.pair_off, q >> 4, q & 15);
    int sg = 0;
    while (sg + 1 < a.nseg && row >= a.n0[sg + 1]) ++sg;
    static_cast<float*>(a.dst)[q] =
        static_cast<const float*>(a.src[sg])[row - a.n0[sg]];
  }
}

template <typename T, int AP, bool WF8>
hipError_t launch_gemm_t(const GemmPlan& pl, const GemmArgs& a, hipStream_t s) {
  dim3 grid(pl.gx, pl.gy, 1), block(pl.waves * 64);
  if (pl.MT == 1 && a.ep == EP_TOP2)
    launch_k((gemm_kernel<T, 1, AP, DFLASH_LM_W, DFLASH_LM_U, false, false,
                          WF8>),
             grid, block, 0, s, a);
  else if (pl.MT == 1)
    launch_k((gemm_kernel<T, 1, AP, DFLASH_GEMM_W, DFLASH_GEMM_U, true,
                          AP == 1, WF8>),
             grid, block, 0, s, a);
  else if (pl.MT == 2)
    launch_k((gemm_kernel<T, 2, AP, 4, 8, true, false, WF8>), grid, block, 0,
             s, a);
  else if (pl.MT == 4)
    launch_k((gemm_kernel<T, 4, AP, 16, 2, true, false, WF8>), grid, block,
             0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int M, int N, bool lm_head) {
  GemmPlan pl;
  pl.MT = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  pl.waves = pl.MT == 1 ? (lm_head ? DFLASH_LM_W : DFLASH_GEMM_W)
                        : (pl.MT == 2 ? 4 : 16);
  pl.gx = N / 16;
  pl.gy = (M + 16 * pl.MT - 1) / (16 * pl.MT);
  return pl;
}

hipError_t launch_gemm(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                       hipStream_t s) {
  if (a.wfp8) {
    // FP8 step pairs: bf16 activations, packed, contraction in whole pairs
    if (!bf16 || !a.a_packed || a.Kd % 64 != 0) return hipErrorInvalidValue;
    return launch_gemm_t<bf16_t, 1, true>(pl, a, s);
  }
  if (bf16)
    return a.a_packed ? launch_gemm_t<bf16_t, 1, false>(pl, a, s)
                      : launch_gemm_t<bf16_t, 0, false>(pl, a, s);
  return a.a_packed ? launch_gemm_t<float, 1, false>(pl, a, s)
                    : launch_gemm_t<float, 0, false>(pl, a, s);
}

constexpr int kLmW = DFLASH_LMP_W, kLmNS = DFLASH_LMP_NS;

int lm_head_parts(bool bf16, int M, int N, int Kd, int num_cu) {
  const int KC = bf16 ? Storage<bf16_t>::KC : Storage<float>::KC;
  if (M > 16 || Kd % KC != 0 || Kd / KC > kLmW * kLmNS) return 0;
  return min(num_cu, N / 16);
}

hipError_t launch_lm_head(bool bf16, int parts, const GemmArgs& a,
                          hipStream_t s) {
  if (parts <= 0 || !a.a_packed) return hipErrorInvalidValue;
  // row scales come with FP8 weights only (and always with them)
  if ((a.wscale != nullptr) != (a.wfp8 != 0)) return hipErrorInvalidValue;
  if (a.wfp8) {
    if (!bf16 || a.Kd % 64 != 0) return hipErrorInvalidValue;
    launch_k((lm_head_kernel<bf16_t, kLmW, kLmNS, true>), dim3(parts),
             dim3(64 * kLmW), 0, s, a);
  } else if (bf16) {
    launch_k((lm_head_kernel<bf16_t, kLmW, kLmNS, false>), dim3(parts),
             dim3(64 * kLmW), 0, s, a);
  } else {
    launch_k((lm_head_kernel<float, kLmW, kLmNS, false>), dim3(parts),
             dim3(64 * kLmW), 0, s, a);
  }
  return hipGetLastError();
}

int proj_stream_parts(bool bf16, const GemmArgs& a, int num_cu) {
  constexpr int KC = Storage<bf16_t>::KC;
  if (!bf16 || !a.wfp8 || !a.a_packed || a.ep != EP_SWIGLU ||
      a.cmap != MAP_PAIRS || a.M > 16 || a.Kd % 64 != 0 ||
      a.Kd / KC > kLmW * kLmNS || num_cu <= 0)
    return 0;
  const int ntiles = a.N / 16;
  if (ntiles < DFLASH_PROJ_STREAM_MIN * num_cu) return 0;
  const int parts = min(num_cu, ntiles);
  return (ntiles + parts - 1) / parts <= kProjMaxTiles ? parts : 0;
}

hipError_t launch_proj_stream(bool bf16, int parts, const GemmArgs& a,
                              hipStream_t s) {
  if (!bf16 || !a.wfp8 || a.wscale == nullptr || parts <= 0 ||
      !a.a_packed || a.ep != EP_SWIGLU || a.cmap != MAP_PAIRS || a.M > 16 ||
      a.Kd % 64 != 0 || a.Kd / Storage<bf16_t>::KC > kLmW * kLmNS ||
      (a.N / 16 + parts - 1) / parts > kProjMaxTiles)
    return hipErrorInvalidValue;
  launch_k((gemm_stream_kernel<kLmW, kLmNS>), dim3(parts), dim3(64 * kLmW),
           0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(bool bf16, const PackArgs& a, hipStream_t s) {
  if (a.mode == PACK_SCALE) {
    launch_k(pack_scale_kernel, dim3((a.N + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (a.mode == PACK_FP8 || a.mode == PACK_FP8_BF16) {
    if (!bf16 || a.K % 64 != 0) return hipErrorInvalidValue;
    const int64_t chunks =
        (int64_t)a.N / 16 * (a.mode == PACK_FP8 ? a.K / 64 : a.K / 32) * 64;
    int64_t blocks = (chunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    launch_k(pack_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int E = bf16 ? Storage<bf16_t>::E : Storage<float>::E;
  const int64_t chunks = (int64_t)a.N * a.K / E;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    launch_k(pack_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    launch_k(pack_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dflash
