// Block attention: the K = 16 block queries of every query head attend to all
// L_b injected context keys plus the K block keys, with no mask.
//
// One workgroup per (context chunk, kv head, sequence); its waves are the
// query heads sharing that kv head (GQA group), each owning its 16 block
// queries.  K and V tiles of 64 keys are staged once in LDS for all waves:
// bf16 tiles go straight from global memory into a ring of tile slots in
// LDS (attn_bf16_kernel), fp32 tiles through two register sets in flight
// (attn_f32_kernel).  The P.V product contracts over keys, so its MFMA
// operand needs several keys of one channel per lane: bf16 V is stored
// key-major like K and read back transposed by the LDS transpose read, fp32
// V is transposed as it is written.  Each wave computes S^T = K Q^T with
// MFMA, keeps an online softmax per query in its own lanes, and accumulates
// O^T = V^T P^T.  Chunks write unnormalised partial outputs with their
// running max and sum; a merge kernel combines the chunks of a sequence in
// chunk order.
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kKeyTile = 64;

// Accuracy of P.V: P is split into DFLASH_ATTN_PSPLIT bf16 parts (2: ~16
// significant bits, 3: exact fp32) and the MFMAs accumulate in fp32 into the
// running output.  Rounding P to a single bf16 part measurably moves the
// drafted logits; more than two parts, or float64 running sums, do not (the
// bf16 rounding of the attention output dominates).
#ifndef DFLASH_ATTN_PSPLIT
#define DFLASH_ATTN_PSPLIT 2
#endif
constexpr int kVPad = 4;  // elements of padding per transposed V row

// LDS transpose read of 16-bit elements (gfx950).  Within each group of 16
// lanes, lane i receives element i % 4 of the 8 bytes read by lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of its group, in that order.  So
// when lane 4e + q of a group points at channels c + 4q .. c + 4q + 3 of key
// k_e, lane i receives channel c + i of keys k_0 .. k_3.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// fp32 form.  Each thread carries NP 16-byte pieces of K and of V for one
// 64-key tile.  Two such register sets are in flight: while tile t is
// computed from LDS, tiles t + 1 and t + 2 are being loaded.
template <typename T, int D, int G>
struct TileRegs {
  static constexpr int PIECES = D / Storage<T>::E;  // 16-byte pieces per key
  static constexpr int NP = kKeyTile * PIECES / (64 * G);
  u32x4 k[NP], v[NP];
};

// Loads are unconditional: keys past the chunk read the chunk's last key
// (finite values whose scores are masked to -inf, so P = 0 for them).
template <typename T, int D, int G>
__device__ __forceinline__ void load_tile(TileRegs<T, D, G>& t, const char* kb,
                                          const char* vb, int kt, int last_key,
                                          int tid) {
  constexpr int SZ = sizeof(T), E = Storage<T>::E;
  constexpr int PIECES = TileRegs<T, D, G>::PIECES;
#pragma unroll
  for (int j = 0; j < TileRegs<T, D, G>::NP; ++j) {
    const int idx = tid + j * 64 * G;
    const int key = min(kt + idx / PIECES, last_key), pc = idx % PIECES;
    const int64_t off = ((int64_t)key * D + pc * E) * SZ;
    t.k[j] = stage_load(kb + off);
    t.v[j] = stage_load(vb + off);
  }
}

// Register sets of K/V tiles in flight (each 2 * NP loads per thread) for
// groups of four or more query heads; groups of two hold twice the pieces
// per thread and keep two sets.
#ifndef DFLASH_ATTN_SETS
#define DFLASH_ATTN_SETS 2
#endif
template <int G>
constexpr int attn_sets() {
  return G >= 4 ? DFLASH_ATTN_SETS : 2;
}
static_assert(DFLASH_ATTN_SETS == 2 || DFLASH_ATTN_SETS == 3,
              "two or three register sets");

// Wait for the oldest register set: the other sets' loads were issued
// after it.
template <typename T, int D, int G>
__device__ __forceinline__ void wait_tile(TileRegs<T, D, G>& t) {
  constexpr int NP = TileRegs<T, D, G>::NP;
  constexpr int AHEAD = (attn_sets<G>() - 1) * 2 * NP;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    vm_wait<AHEAD>(t.k[j]);
    vm_wait<AHEAD>(t.v[j]);
  }
}

// (at four waves, two workgroups per compute unit: at most 256 VGPRs)
template <int D, int G>
__global__ __launch_bounds__(64 * G, G == 4 ? 2 : 1) void attn_f32_kernel(
    AttnArgs p) {
  using T = float;
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC, SZ = sizeof(T);
  constexpr int DC = D / KC;
  // padded K row (bytes): the 16 rows of a score read cover every bank once
  constexpr int KROWB = D * SZ + 16;
  constexpr int VROW = kKeyTile + kVPad;       // transposed V row, elements
  constexpr int VROWB = VROW * SZ;
  constexpr int PIECES = TileRegs<T, D, G>::PIECES;
  constexpr int NP = TileRegs<T, D, G>::NP;
  constexpr int VBYTES = D * VROWB;            // V in LDS, transposed
  static_assert(NP * 64 * G == kKeyTile * PIECES, "tile pieces per thread");
  // K and V tiles, double-buffered by tile parity
  __shared__ __attribute__((aligned(16))) char ks2[2][kKeyTile * KROWB];
  __shared__ __attribute__((aligned(16))) char vt2[2][VBYTES];

  constexpr int kSets = attn_sets<G>();
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  // one value for the workgroup: the tile positions (and page lookups)
  // derived from it stay scalar
  int L = __builtin_amdgcn_readfirstlane(p.ctx_len[b]);
  L = min(max(L, 0), p.max_len);
  const int nkeys = L + p.K;
  const int k0 = c * p.chunk;
  if (k0 >= nkeys) return;
  const int k1 = min(nkeys, k0 + p.chunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int hq = kvh * G + wave;

  // K/V of the 64-key tile at kt: load_tile adds key * D to these bases.
  // A tile never straddles a page (pages hold a multiple of 64 positions);
  // a tile past the chunk's end reads the chunk's last key, so its page is
  // the last key's.
  auto load_at = [&](TileRegs<T, D, G>& t, int kt) {
    const int pk = min(kt, k1 - 1);
    const int first = p.pages.log2 < 0 ? 0 : (pk >> p.pages.log2) << p.pages.log2;
    const int64_t off =
        (kv_row_uniform(p.pages, p.P, p.Hkv, b, kvh, first, p.err) - first) *
        D * SZ;
    load_tile<T, D, G>(t, static_cast<const char*>(p.kc) + off,
                       static_cast<const char*>(p.vc) + off, kt, k1 - 1, tid);
  };
  // Q fragments of this wave's head: lane (query r, group g).  They are
  // staging loads issued ahead of the K/V prefetch and waited for once
  // below: a compiler-tracked load would make each use inside the tile loop
  // wait for every load then in flight, draining the prefetch at each tile.
  const char* qrow = static_cast<const char*>(p.q) +
                     ((int64_t)(b * p.K + r) * p.Hq * D + hq * D + g * E) * SZ;
  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = stage_load(qrow + dc * KC * SZ);
  TileRegs<T, D, G> regs0, regs1, regs2;
  load_at(regs0, k0);
  load_at(regs1, k0 + kKeyTile);
  if constexpr (kSets == 3) load_at(regs2, k0 + 2 * kKeyTile);
  stage_wait<0, DC, kSets * 2 * NP>(qf);

  // running max (log2 domain), softmax numerator o and denominator l
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 64-key tile at kt from register set rg, which is then refilled with
  // the tile kSets ahead
  auto step = [&](TileRegs<T, D, G>& rg, int kt) {
    wait_tile<T, D, G>(rg);
    // buffer (tile index) % 2: its readers two tiles back are done, since
    // every wave has passed the previous tile's barrier
    const int buf = ((kt - k0) / kKeyTile) & 1;
    char* ks = ks2[buf];
    char* vt = vt2[buf];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int idx = tid + j * 64 * G;
      const int key = idx / PIECES, pc = idx % PIECES;
      *reinterpret_cast<u32x4*>(ks + key * KROWB + pc * E * SZ) = rg.k[j];
      const T* ve = reinterpret_cast<const T*>(&rg.v[j]);
      T* vcol = reinterpret_cast<T*>(vt) + key;
#pragma unroll
      for (int e = 0; e < E; ++e) vcol[(pc * E + e) * VROW] = ve[e];
    }
    __syncthreads();
    load_at(rg, kt + kSets * kKeyTile);
    if (kt >= k1) return;  // past the chunk's last tile: nothing to compute
    const int n_valid = min(kKeyTile, k1 - kt);

    // S^T tile: rows = 64 keys (4 MFMA row tiles), columns = 16 queries
    f32x4 s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const char* krow = ks + (16 * mt + r) * KROWB + g * E * SZ;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        mma16(s[mt], load16(krow + dc * KC * SZ), qf[dc], T());
    }
    // online softmax for query r (log2 domain); keys 16mt + 4g + j (only a
    // chunk's last tile can hold keys past its end: a uniform branch)
    float tmax = -INFINITY;
    if (n_valid == kKeyTile) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[mt][j] *= p.scale_log2;
          tmax = fmaxf(tmax, s[mt][j]);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = 16 * mt + 4 * g + j;
          const float v = key < n_valid ? s[mt][j] * p.scale_log2 : -INFINITY;
          s[mt][j] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    // the same factor scales numerator and denominator, so its rounding
    // cancels in o = numerator / denominator; once the running maxima have
    // settled the factor is 1 for every query and the rescale is skipped
    // The hardware exp2 (no rescaling for results below 2^-126, which it
    // flushes: such weights add nothing a float32 sum of values near 1 keeps)
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lt = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(s[mt][j] - m_new);
        s[mt][j] = pv;
        lt += pv;
      }
    l_run = l_run * alpha + lt;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[dt][j] *= alpha;
    }

    // O^T += V^T P^T; contraction slots of lane group g hold the keys that
    // this lane's S^T registers hold
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const u32x4 bfrag = {__float_as_uint(s[cc][0]), __float_as_uint(s[cc][1]),
                           __float_as_uint(s[cc][2]), __float_as_uint(s[cc][3])};
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const char* vrow = vt + (16 * dt + r) * VROWB;
        const u32x4 afrag = *reinterpret_cast<const u32x4*>(vrow + (16 * cc + 4 * g) * SZ);
        mma16(o[dt], afrag, bfrag, T());
      }
    }
  };
  for (int kt = k0; kt < k1; kt += kSets * kKeyTile) {
    step(regs0, kt);
    step(regs1, kt + kKeyTile);
    if constexpr (kSets == 3) step(regs2, kt + 2 * kKeyTile);
  }
  // the last refills are still in flight: wait before the registers die
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    vm_wait<0>(regs0.k[j]);
    vm_wait<0>(regs0.v[j]);
    vm_wait<0>(regs1.k[j]);
    vm_wait<0>(regs1.v[j]);
    if constexpr (kSets == 3) {
      vm_wait<0>(regs2.k[j]);
      vm_wait<0>(regs2.v[j]);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (p.nch == 1) {
    // One chunk holds the whole softmax: normalise here with the merge's
    // arithmetic (float64 quotient, one rounding to the storage type, the
    // same bits) and write the packed output; no merge runs.
    const double inv = 1.0 / (double)l_tot;
    const int row = b * p.K + r, Kd = p.Hq * D;
    char* ob = static_cast<char*>(p.o);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      char* dst = ob + packed_offset<T>(row, hq * D + 16 * dt + 4 * g, Kd);
      u32x4 w;
      T* wt = reinterpret_cast<T*>(&w);
#pragma unroll
      for (int e = 0; e < 4; ++e) store_elem(wt, e, (double)o[dt][e] * inv);
      *reinterpret_cast<u32x4*>(dst) = w;
    }
    return;
  }
  // partials are chunk-major within (sequence, query head, query):
  // part_o[((b*Hq + hq)*K + i)*nch + c][D], part_ml[... same index][2]
  const int64_t base = (((int64_t)b * p.Hq + hq) * p.K + r) * p.nch + c;
  float* po = p.part_o + base * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
  if (g == 0)
    *reinterpret_cast<float2*>(p.part_ml + base * 2) = float2{m_run, l_tot};
}

// bf16 form: K and V tiles go from global memory straight into a ring
// of NBUF tile slots in LDS (global_load_lds_dwordx4: lane l's 16 bytes
// land at m0 + 16 l), so no registers stage them and no LDS stores copy
// them; NBUF - 1 tiles are in flight while one is computed.  Rows are not
// padded: the 16-byte pieces of key k are stored permuted (piece p at
// position p ^ swz(k)), the DMA lanes fetching the pieces that belong at
// their positions, so that the score reads (16 keys at one piece) and the
// transposed V reads (8 keys at two adjacent pieces) hit every bank once.
// (the scalar-base form: a wave-uniform 64-bit base in SGPRs plus this
// lane's 32-bit byte offset, so a load costs no vector address arithmetic)
__device__ __forceinline__ void attn_lds_load16(const char* base, uint32_t off,
                                                uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void attn_vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// piece permutations (SPR 16-byte pieces per key row: 16 for d = 128, 8
// for d = 64; a 256-byte bank window holds 256 / (16 SPR) rows)
template <int SPR>
__device__ __forceinline__ int swz_k(int key) {
  return (key / (16 / SPR)) & (SPR - 1);
}
template <int SPR>
__device__ __forceinline__ int swz_v(int key) {
  return 2 * ((key / (16 / SPR)) & (SPR / 2 - 1));
}

// The sequence whose context is the z-th longest of the B in the batch
// (equal lengths: lower index first), for a grid that runs sequences
// longest first.  Every thread of the workgroup calls it (one barrier).
__device__ int seq_by_length_rank(const AttnArgs& p, int z, int B) {
  __shared__ int pick;
  auto len = [&](int s) { return min(max(p.ctx_len[s], 0), p.max_len); };
  for (int s = threadIdx.x; s < B; s += blockDim.x) {
    const int ls = len(s);
    int rank = 0;
    for (int u = 0; u < B; ++u) {
      const int lu = len(u);
      rank += (lu > ls) || (lu == ls && u < s);
    }
    if (rank == z) pick = s;
  }
  __syncthreads();
  return pick;
}

template <int D, int G, int NBUF>
__global__ __launch_bounds__(64 * G, G == 4 && NBUF <= 2 ? 2 : 1) void
attn_bf16_kernel(AttnArgs p) {
  using T = bf16_t;
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC, SZ = sizeof(T);
  constexpr int DC = D / KC;
  constexpr int SPR = D / E;                  // pieces per key row
  constexpr int TB = kKeyTile * D * SZ;       // bytes of one K (or V) tile
  constexpr int NI = TB / 1024;               // 1 KiB loads per tile and operand
  constexpr int IPW = NI / G;                 // ... per wave
  constexpr int LPT = 2 * IPW;                // loads per wave per tile
  static_assert(IPW * G == NI, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char ring[NBUF][2][TB];

  const int c = blockIdx.x, kvh = blockIdx.y;
  // with one chunk per sequence the grid takes the sequences longest first,
  // so that the workgroups sharing a CU pair long contexts with short ones
  const int b = __builtin_amdgcn_readfirstlane(
      p.by_len ? seq_by_length_rank(p, blockIdx.z, gridDim.z)
               : (int)blockIdx.z);
  int L = __builtin_amdgcn_readfirstlane(p.ctx_len[b]);
  L = min(max(L, 0), p.max_len);
  const int nkeys = L + p.K;
  const int k0 = c * p.chunk;
  if (k0 >= nkeys) return;
  const int k1 = min(nkeys, k0 + p.chunk);
  const int ntile = (k1 - k0 + kKeyTile - 1) / kKeyTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int hq = kvh * G + wave;
  const uint32_t lds0 =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ring;

  // this lane's part of load i (of IPW) of a tile: key row within the tile
  // and the byte offset of its piece, for K and for V (the same keys,
  // other pieces)
  int key_of[IPW], koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int slot = (wave + i * G) * 64 + lane;
    const int key = slot / SPR, q = slot % SPR;
    key_of[i] = key;
    koff[i] = (q ^ swz_k<SPR>(key)) * 16;
    voff[i] = (q ^ swz_v<SPR>(key)) * 16;
  }
  // tile j of the chunk into ring slot j % NBUF.  A tile never straddles a
  // page (pages hold a multiple of 64 positions), so its rows lie at one
  // wave-uniform base; keys past the chunk read its last key (finite values
  // whose scores are masked, so P = 0).
  auto issue = [&](int j) {
    const int kt = k0 + j * kKeyTile;
    const int first = p.pages.log2 < 0 ? 0 : (kt >> p.pages.log2) << p.pages.log2;
    const int64_t rowb =
        (kv_row_uniform(p.pages, p.P, p.Hkv, b, kvh, first, p.err) - first +
         kt) * (int64_t)D * SZ;
    const char* kb = static_cast<const char*>(p.kc) + rowb;
    const char* vb = static_cast<const char*>(p.vc) + rowb;
    const int lim = k1 - 1 - kt;  // last key of the chunk, from the tile
    const uint32_t sl = lds0 + (uint32_t)((j % NBUF) * 2 * TB);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const uint32_t row = (uint32_t)(min(key_of[i], lim) * (D * SZ));
      const uint32_t at = (uint32_t)((wave + i * G) * 1024);
      attn_lds_load16(kb, row + koff[i], sl + at);
      attn_lds_load16(vb, row + voff[i], sl + TB + at);
    }
  };

  // Q fragments of this wave's head: staging loads, waited for once below.
  // The first NBUF - 1 tiles are issued in straight-line code whatever the
  // chunk's length (a chunk of fewer tiles loads its last tile again, into
  // that tile's own slot), so that the wait sits at one point with one
  // count: a branch here would let the compiler copy the Q registers, at
  // the join, before their loads have landed.
  const char* qrow = static_cast<const char*>(p.q) +
                     ((int64_t)(b * p.K + r) * p.Hq * D + hq * D + g * E) * SZ;
  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = stage_load(qrow + dc * KC * SZ);
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j) issue(min(j, ntile - 1));
  stage_wait<0, DC, (NBUF - 1) * LPT>(qf);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < ntile; ++j) {
    // this wave's loads of tile j have landed (NBUF - 2 later tiles may
    // still be in flight; near the end, fewer were issued: wait for all)
    if (j + NBUF - 2 < ntile)
      attn_vm_wait<(NBUF - 2) * LPT>();
    else
      attn_vm_wait<0>();
    // every wave's part of tile j is visible, and every wave has finished
    // tile j - 1, whose slot is refilled with tile j + NBUF - 1
    __syncthreads();
    if (j + NBUF - 1 < ntile) issue(j + NBUF - 1);
    const char* ks = ring[j % NBUF][0];
    const char* vt = ring[j % NBUF][1];
    const int kt = k0 + j * kKeyTile;
    const int n_valid = min(kKeyTile, k1 - kt);

    // S^T tile: rows = 64 keys (4 MFMA row tiles), columns = 16 queries
    f32x4 s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = 16 * mt + r;
      const char* krow = ks + key * (D * SZ);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        mma16(s[mt], load16(krow + ((g + 4 * dc) ^ swz_k<SPR>(key)) * 16),
              qf[dc], T());
    }
    // online softmax for query r (log2 domain); keys 16mt + 4g + j (only a
    // chunk's last tile can hold keys past its end: a uniform branch)
    float tmax = -INFINITY;
    if (n_valid == kKeyTile) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          s[mt][jj] *= p.scale_log2;
          tmax = fmaxf(tmax, s[mt][jj]);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = 16 * mt + 4 * g + jj;
          const float v = key < n_valid ? s[mt][jj] * p.scale_log2 : -INFINITY;
          s[mt][jj] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float lt = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pv = __builtin_amdgcn_exp2f(s[mt][jj] - m_new);
        s[mt][jj] = pv;
        lt += pv;
      }
    l_run = l_run * alpha + lt;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) o[dt][jj] *= alpha;
    }

    // O^T += V^T P^T with P = p1 + p2 (+ p3) in bf16 parts
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      constexpr int NP3 = DFLASH_ATTN_PSPLIT;
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      float rem[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rem[e] = s[2 * cc + e / 4][e % 4];
      u32x4 bp[NP3];
#pragma unroll
      for (int t = 0; t < NP3; ++t) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x2_t h = {(__bf16)rem[2 * q], (__bf16)rem[2 * q + 1]};
          w[q] = __builtin_bit_cast(uint32_t, h);
          rem[2 * q] -= __uint_as_float(w[q] << 16);
          rem[2 * q + 1] -= __uint_as_float(w[q] & 0xFFFF0000u);
        }
        bp[t] = u32x4{w[0], w[1], w[2], w[3]};
      }
      // lane (r, g) reads 8 bytes of key 32cc + 4g + r/4 (+16): channels
      // 16dt + 4(r%4) .. +3, piece 2dt + (r%4)/2 of the row, and receives
      // channel 16dt + r of keys 32cc + 4g + 0..3 (lo) and +16 (hi)
      const int klo = 32 * cc + 4 * g + (r >> 2), khi = klo + 16;
      const char* vlo = vt + klo * (D * SZ) + (r & 1) * 8;
      const char* vhi = vt + khi * (D * SZ) + (r & 1) * 8;
      const int sl = swz_v<SPR>(klo), sh = swz_v<SPR>(khi);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int pc = 2 * dt + ((r & 3) >> 1);
        const u32x2 lo = lds_read_tr16(vlo + (pc ^ sl) * 16);
        const u32x2 hi = lds_read_tr16(vhi + (pc ^ sh) * 16);
        const u32x4 afrag = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int t = 0; t < NP3; ++t) mma16(o[dt], afrag, bp[t], T());
      }
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (p.nch == 1) {
    // one chunk holds the whole softmax: normalise here with the merge's
    // arithmetic (float64 quotient, one rounding) and write the packed output
    const double inv = 1.0 / (double)l_tot;
    const int row = b * p.K + r, Kd = p.Hq * D;
    char* ob = static_cast<char*>(p.o);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      char* dst = ob + packed_offset<T>(row, hq * D + 16 * dt + 4 * g, Kd);
      u32x2 w;
      T* wt = reinterpret_cast<T*>(&w);
#pragma unroll
      for (int e = 0; e < 4; ++e) store_elem(wt, e, (double)o[dt][e] * inv);
      *reinterpret_cast<u32x2*>(dst) = w;
    }
    return;
  }
  const int64_t base = (((int64_t)b * p.Hq + hq) * p.K + r) * p.nch + c;
  float* po = p.part_o + base * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4*>(po + 16 * dt + 4 * g) = o[dt];
  if (g == 0)
    *reinterpret_cast<float2*>(p.part_ml + base * 2) = float2{m_run, l_tot};
}

// o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the sequence's
// chunks (M = the largest m_c), written packed for the output projection.
// One wave per (sequence, query head, block query): lane c reads chunk c's
// (m, l) so the weights come from wave reductions (fixed butterfly order);
// the partial outputs are then summed in chunk order, lane owning D/64
// consecutive channels, with MB chunks' loads in flight (the grid's chunk
// count rounded up to a multiple of 4, at most 32, so few chunks do not
// issue loads that repeat the last one).  The sums run in chunk order
// whatever MB is.
template <typename T, int D, int MB>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p, int rows) {
  constexpr int DPL = D / 64;
  const int wrow = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wrow >= rows) return;
  const int lane = threadIdx.x & 63;
  const int i = wrow % p.K, bh = wrow / p.K;
  const int b = bh / p.Hq, hq = bh % p.Hq;
  int L = p.ctx_len[b];
  L = min(max(L, 0), p.max_len);
  const int nc = (L + p.K + p.chunk - 1) / p.chunk;
  const int64_t base = (int64_t)wrow * p.nch;  // == ((b*Hq + hq)*K + i)*nch
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + base;
  const float* ob = p.part_o + base * D + lane * DPL;

  // The first batch of partial outputs does not depend on the weights:
  // issue its loads before the reductions.  Every row has nch chunk slots,
  // so the loads are made unconditionally (clamped to the slots, not to the
  // row's own chunk count, which needs ctx_len first) and the values of
  // chunks past nc are dropped below.
  float v[MB][DPL];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int c = min(c0 + u, p.nch - 1);
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = ob[(int64_t)c * D + e];
    }
  };
  load_batch(0);
  // chunk weights 2^(m_c - M): lane c holds chunk c (c < 64); further
  // chunks, if any, are read again where needed
  const float2 t_l = ml[min(lane, p.nch - 1)];
  const float m_l = lane < nc ? t_l.x : -INFINITY;
  const float l_l = lane < nc ? t_l.y : 0.f;
  float M = m_l;
  for (int c = lane + 64; c < nc; c += 64) M = fmaxf(M, ml[c].x);
  M = warp_max(M);
  const float w_l = lane < nc ? exp2f(m_l - M) : 0.f;
  double ls = (double)w_l * (double)l_l;
  for (int c = lane + 64; c < nc; c += 64)
    ls += (double)exp2f(ml[c].x - M) * (double)ml[c].y;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);

  double acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
  for (int c0 = 0; c0 < nc; c0 += MB) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int c = c0 + u;  // uniform across the wave
      if (c < nc) {
        const float w = c < 64 ? __shfl(w_l, c, 64) : exp2f(ml[c].x - M);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += (double)w * (double)v[u][e];
      }
    }
  }
  const double inv = 1.0 / ls;
  const int row = b * p.K + i, Kd = p.Hq * D, d0 = lane * DPL;
  T* dst = reinterpret_cast<T*>(static_cast<char*>(p.o) +
                                packed_offset<T>(row, hq * D + d0, Kd));
#pragma unroll
  for (int e = 0; e < DPL; ++e) store_elem(dst, e, acc[e] * inv);
}

// ring slots of the bf16 kernel: two workgroups per CU (about 2 x 64 KiB of
// LDS with d = 128) or one (deep: chunks of 2048+ keys)
#ifndef DFLASH_ATTN_RING
#define DFLASH_ATTN_RING 2
#endif
#ifndef DFLASH_ATTN_RING_DEEP
#define DFLASH_ATTN_RING_DEEP 4
#endif
template <typename T, int D, int G>
hipError_t attn_t(int B, const AttnArgs& a, hipStream_t s) {
  const dim3 agrid(a.nch, a.Hkv, B);
  if constexpr (sizeof(T) == 2) {
    if (a.deep)
      launch_k((attn_bf16_kernel<D, G, DFLASH_ATTN_RING_DEEP>), agrid,
               dim3(64 * G), 0, s, a);
    else
      launch_k((attn_bf16_kernel<D, G, DFLASH_ATTN_RING>), agrid, dim3(64 * G),
               0, s, a);
  } else {
    launch_k((attn_f32_kernel<D, G>), agrid, dim3(64 * G), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nch == 1) return hipSuccess;  // the partial kernel normalised
  const int rows = B * a.Hq * a.K;
  const dim3 grid((rows + 3) / 4), block(256);
  switch (a.nch <= 32 ? (a.nch + 3) / 4 : 8) {
    case 1: launch_k((attn_merge_kernel<T, D, 4>), grid, block, 0, s, a, rows); break;
    case 2: launch_k((attn_merge_kernel<T, D, 8>), grid, block, 0, s, a, rows); break;
    case 3: launch_k((attn_merge_kernel<T, D, 12>), grid, block, 0, s, a, rows); break;
    case 4: launch_k((attn_merge_kernel<T, D, 16>), grid, block, 0, s, a, rows); break;
    case 5: launch_k((attn_merge_kernel<T, D, 20>), grid, block, 0, s, a, rows); break;
    case 6: launch_k((attn_merge_kernel<T, D, 24>), grid, block, 0, s, a, rows); break;
    case 7: launch_k((attn_merge_kernel<T, D, 28>), grid, block, 0, s, a, rows); break;
    default: launch_k((attn_merge_kernel<T, D, 32>), grid, block, 0, s, a, rows); break;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t attn_g(int B, const AttnArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {  // group sizes allowed at create
    case 2: return attn_t<T, D, 2>(B, a, s);
    case 4: return attn_t<T, D, 4>(B, a, s);
    case 8: return attn_t<T, D, 8>(B, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(bool bf16, int d, int B, const AttnArgs& a,
                            hipStream_t s) {
  // fp32 drafters have head_dim 64 (checked at create)
  if (d == 128) return bf16 ? attn_g<bf16_t, 128>(B, a, s) : hipErrorInvalidValue;
  if (d == 64) return bf16 ? attn_g<bf16_t, 64>(B, a, s) : attn_g<float, 64>(B, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dflash
