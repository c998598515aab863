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
// (one 16-row tile); measured on MI355X, see the design notes.
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


// acc[m] over this wave's share of the contraction.  With F64 each MFMA
// step (32 contraction elements) is summed in fp32 from zero and added to a
// float64 accumulator: the projections feed bf16-rounded activations of the
// next step, where fp32 accumulation error over thousands of terms flips
// roundings that then spread through the layer.  The LM head's logits feed
// nothing further and accumulate in fp32.
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
template <int AHEAD, int NL, int U, int MT, typename T, bool F64>
__device__ __forceinline__ void packed_block(u32x4 (&st)[NL], int first,
                                             int n_i, double (&acc)[MT][4],
                                             f32x4 (&acc32)[MT]) {
  stage_wait<0, NL, AHEAD>(st);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (first + u >= n_i) break;  // uniform: past this wave's last step
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if constexpr (F64) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        mma16(t, st[u * (1 + MT) + 1 + m], st[u * (1 + MT)], T());
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] += (double)t[j];
      } else {
        mma16(acc32[m], st[u * (1 + MT) + 1 + m], st[u * (1 + MT)], T());
      }
    }
  }
}

template <typename T, int MT, int W, int U, bool F64>
__device__ __forceinline__ void gemm_core_packed(const GemmArgs& p, int tile,
                                                 int m_base,
                                                 double (&acc)[MT][4]) {
  constexpr int KC = Storage<T>::KC;
  constexpr int NL = U * (1 + MT);  // loads per block: weight, then A tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = p.Kd / KC;
  const char* wbase =
      static_cast<const char*>(p.w) + ((int64_t)tile * nsteps * 64 + lane) * 16;
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
  const int n_i = wave < nsteps ? (nsteps - 1 - wave) / W + 1 : 0;
  const int nb = (n_i + U - 1) / U;
  // block b holds this wave's steps bU .. bU + U - 1 (clamped to the last)
  auto load = [&](u32x4(&st)[NL], int blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(blk * U + u, n_i - 1);
      const int64_t off = (int64_t)(wave + i * W) * 1024;
      st[u * (1 + MT)] = stage_load(wbase + off);
#pragma unroll
      for (int m = 0; m < MT; ++m) st[u * (1 + MT) + 1 + m] = stage_load(abase[m] + off);
    }
  };
  if (nb > 0) {
    // Straight-line shape: both sets loaded, pairs of blocks while a refill
    // exists, then the last pair with no refill.  Every set has a single
    // consumer, so no in-flight register is ever copied.  With an odd block
    // count the last refill of s1 (or, for one block, s1 itself) repeats
    // the wave's last step and is not multiplied.
    u32x4 s0[NL], s1[NL];
    load(s0, 0);
    load(s1, 1);
    int blk = 0;
    for (; blk + 2 < nb; blk += 2) {
      packed_block<NL, NL, U, MT, T, F64>(s0, blk * U, n_i, acc, acc32);
      load(s0, blk + 2);
      packed_block<NL, NL, U, MT, T, F64>(s1, (blk + 1) * U, n_i, acc, acc32);
      load(s1, blk + 3);
    }
    packed_block<NL, NL, U, MT, T, F64>(s0, blk * U, n_i, acc, acc32);
    packed_block<0, NL, U, MT, T, F64>(s1, (blk + 1) * U, n_i, acc, acc32);
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
template <int MT, int W>
__device__ __forceinline__ void reduce_waves(const double (&acc)[MT][4],
                                             double* redd, float* red) {
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
template <typename T, int MT, int AP, int W, int U, bool F64, bool PIPE>
__global__ __launch_bounds__(64 * W) void gemm_kernel(GemmArgs p) {
  static_assert(!PIPE || AP, "the pipelined core reads packed A");
  __shared__ double redd[W * 256];
  __shared__ float red[MT * 256];
  const int tile = blockIdx.x, m_base = blockIdx.y * 16 * MT;
  double acc[MT][4];
  if constexpr (PIPE)
    gemm_core_packed<T, MT, W, U, F64>(p, tile, m_base, acc);
  else
    gemm_core<T, MT, AP, W, U, F64>(p, tile, m_base, acc);
  reduce_waves<MT, W>(acc, redd, red);
  apply_epilogue<T, MT, W>(p, tile, m_base, red);
}

// LM head for up to 16 drafted rows: one persistent workgroup per compute
// unit streams every P-th 16-column vocabulary tile (the workgroups sweep
// the matrix together).  Each wave keeps its share of the activation
// fragments in registers for the workgroup's lifetime, and the weight
// fragments of the next two tiles are in flight in two register sets while
// the current tile is multiplied, summed over the waves and reduced to top-2
// records, so the weight stream does not pause at tile boundaries.  A tile
// is summed exactly as in gemm_kernel (fp32 over a wave's steps, then
// float64 over the waves in wave order); each row's record is merged over
// the workgroup's tiles in tile order and written once per workgroup:
// part[row][workgroup].

// AHEAD: staging loads issued after this tile's set (the other set's, or
// none for the last tile).  The tile is multiplied from set b; with REFILL
// b is then reloaded with the tile two ahead, before the wave sums.
template <typename T, int W, int NS, int AHEAD, bool REFILL, typename LoadW>
__device__ __forceinline__ void lm_tile(const GemmArgs& p, u32x4 (&a)[NS],
                                        u32x4 (&b)[NS], int n_i, int i,
                                        int tile, bool valid, double* redd,
                                        Top2& run, const LoadW& load_w) {
  stage_wait<0, NS, AHEAD>(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < n_i) mma16(acc, a[s], b[s], T());
  if constexpr (REFILL) load_w(b, i + 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) redd[wave * 256 + j * 64 + lane] = (double)acc[j];
  __syncthreads();
  if (threadIdx.x < 256 && valid) {
    const int idx = threadIdx.x;
    // idx = (j, row group, column): row 4 (idx % 64 / 16) + idx / 64
    double v = redd[idx];
#pragma unroll
    for (int w = 1; w < W; ++w) v += redd[w * 256 + idx];
    const float z = (float)v;
    const int row = 4 * ((idx & 63) >> 4) + (idx >> 6);
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

template <typename T, int W, int NS>
__global__ __launch_bounds__(64 * W) void lm_head_kernel(GemmArgs p) {
  constexpr int KC = Storage<T>::KC;
  __shared__ double redd[2][W * 256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nsteps = p.Kd / KC;
  const int ntiles = p.N / 16, P = gridDim.x, wg = blockIdx.x;
  // tiles wg, wg + P, ...: the workgroups sweep the matrix together
  const int nt = (ntiles - 1 - wg) / P + 1;  // >= 1: P <= ntiles
  auto tile_of = [&](int i) { return wg + min(i, nt - 1) * P; };
  // this wave's steps: wave, wave + W, ... (n_i of them, n_i <= NS)
  const int n_i = wave < nsteps ? (nsteps - 1 - wave) / W + 1 : 0;
  const int64_t step_off = (int64_t)wave * 1024 + lane * 16;
  // a step past the wave's last repeats the last (a wave with no steps
  // reads step 0), a slot past the last tile repeats the last tile; neither
  // is multiplied or summed
  auto load_w = [&](u32x4(&b)[NS], int i) {  // this workgroup's i-th tile
    const char* wt = static_cast<const char*>(p.w) +
                     (int64_t)tile_of(i) * nsteps * 1024 + step_off;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      b[s] = stage_load(wt + (int64_t)min(s, max(n_i - 1, 0)) * W * 1024);
  };
  u32x4 a[NS], b0[NS], b1[NS];
  {
    const char* at = static_cast<const char*>(p.a_ptr[0]) + step_off;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      a[s] = stage_load(at + (int64_t)min(s, max(n_i - 1, 0)) * W * 1024);
  }
  load_w(b0, 0);
  load_w(b1, 1);
  stage_wait<0, NS, 2 * NS>(a);
  Top2 run = top2_empty();
  int i = 0;
  for (; i + 2 < nt; i += 2) {
    lm_tile<T, W, NS, NS, true>(p, a, b0, n_i, i, tile_of(i), true, redd[0],
                                run, load_w);
    lm_tile<T, W, NS, NS, true>(p, a, b1, n_i, i + 1, tile_of(i + 1), true,
                                redd[1], run, load_w);
  }
  lm_tile<T, W, NS, NS, false>(p, a, b0, n_i, i, tile_of(i), true, redd[0],
                               run, load_w);
  // the second set was loaded whether or not its tile exists: wait for it
  // either way (only its sums are skipped)
  lm_tile<T, W, NS, 0, false>(p, a, b1, n_i, i + 1, tile_of(i + 1), i + 1 < nt,
                              redd[1], run, load_w);
  if (threadIdx.x < 256 && (threadIdx.x & 15) == 0) {
    const int row = 4 * ((threadIdx.x & 63) >> 4) + (threadIdx.x >> 6);
    if (row < p.M) p.top2[(int64_t)row * P + wg] = run;
  }
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

template <typename T, int AP>
hipError_t launch_gemm_t(const GemmPlan& pl, const GemmArgs& a, hipStream_t s) {
  dim3 grid(pl.gx, pl.gy, 1), block(pl.waves * 64);
  if (pl.MT == 1 && a.ep == EP_TOP2)
    launch_k(
        (gemm_kernel<T, 1, AP, DFLASH_LM_W, DFLASH_LM_U, false, false>), grid,
        block, 0, s, a);
  else if (pl.MT == 1)
    launch_k((gemm_kernel<T, 1, AP, DFLASH_GEMM_W, DFLASH_GEMM_U,
                                    true, AP == 1>),
                       grid, block, 0, s, a);
  else if (pl.MT == 2)
    launch_k((gemm_kernel<T, 2, AP, 4, 8, true, false>), grid, block,
                       0, s, a);
  else if (pl.MT == 4)
    launch_k((gemm_kernel<T, 4, AP, 16, 2, true, false>), grid,
                       block, 0, s, a);
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
  if (bf16)
    return a.a_packed ? launch_gemm_t<bf16_t, 1>(pl, a, s)
                      : launch_gemm_t<bf16_t, 0>(pl, a, s);
  return a.a_packed ? launch_gemm_t<float, 1>(pl, a, s)
                    : launch_gemm_t<float, 0>(pl, a, s);
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
  if (bf16)
    launch_k((lm_head_kernel<bf16_t, kLmW, kLmNS>), dim3(parts),
                       dim3(64 * kLmW), 0, s, a);
  else
    launch_k((lm_head_kernel<float, kLmW, kLmNS>), dim3(parts),
                       dim3(64 * kLmW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(bool bf16, const PackArgs& a, hipStream_t s) {
  const int E = bf16 ? Storage<bf16_t>::E : Storage<float>::E;
  const int64_t chunks = (int64_t)a.N * a.K / E;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    launch_k(pack_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0,
                       s, a);
  else
    launch_k(pack_kernel<float>, dim3((unsigned)blocks), dim3(256), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace dflash
