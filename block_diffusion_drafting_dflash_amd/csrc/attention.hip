// Block attention: the K = 16 block queries of every query head attend to all
// L_b injected context keys plus the K block keys, with no mask.
//
// One workgroup per (context chunk, kv head, sequence); its waves are the
// query heads sharing that kv head (GQA group), each owning its 16 block
// queries.  K and V tiles of 64 keys are staged once in LDS for all waves
// (V transposed so the P.V product can use MFMA with keys as the contraction
// index).  Each wave computes S^T = K Q^T with MFMA, keeps an online softmax
// per query in its own lanes, and accumulates O^T = V^T P^T.  Chunks write
// unnormalised partial outputs with their running max and sum; a merge
// kernel combines the chunks of a sequence in chunk order.
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kKeyTile = 64;
constexpr int kVPad = 4;  // elements of padding per transposed V row

template <typename T, int D>
__global__ __launch_bounds__(512) void attn_partial_kernel(AttnArgs p) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC, SZ = sizeof(T);
  constexpr int DC = D / KC;
  constexpr int KROWB = D * SZ + 16;           // padded K row, bytes
  constexpr int VROW = kKeyTile + kVPad;       // transposed V row, elements
  constexpr int VROWB = VROW * SZ;
  constexpr int PIECES = D / E;                // 16-byte pieces per key row
  __shared__ __attribute__((aligned(16))) char ks[kKeyTile * KROWB];
  __shared__ __attribute__((aligned(16))) char vt[D * VROWB];

  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  int L = p.ctx_len[b];
  L = min(max(L, 0), p.max_len);
  const int nkeys = L + p.K;
  const int k0 = c * p.chunk;
  if (k0 >= nkeys) return;
  const int k1 = min(nkeys, k0 + p.chunk);

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int hq = kvh * G + wave;

  // Q fragments of this wave's head: lane (query r, group g)
  const char* qrow = static_cast<const char*>(p.q) +
                     ((int64_t)(b * p.K + r) * p.Hq * D + hq * D + g * E) * SZ;
  u32x4 qf[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) qf[dc] = load16(qrow + dc * KC * SZ);

  const int64_t head_off = ((int64_t)b * p.Hkv + kvh) * p.P * D;
  const char* kbase = static_cast<const char*>(p.kc) + head_off * SZ;
  const char* vbase = static_cast<const char*>(p.vc) + head_off * SZ;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kt = k0; kt < k1; kt += kKeyTile) {
    const int n_valid = min(kKeyTile, k1 - kt);
    __syncthreads();
    for (int idx = tid; idx < kKeyTile * PIECES; idx += nthr) {
      const int key = idx / PIECES, pc = idx % PIECES;
      u32x4 kv4 = {0u, 0u, 0u, 0u}, vv4 = {0u, 0u, 0u, 0u};
      if (key < n_valid) {
        const int64_t off = ((int64_t)(kt + key) * D + pc * E) * SZ;
        kv4 = load16(kbase + off);
        vv4 = load16(vbase + off);
      }
      *reinterpret_cast<u32x4*>(ks + key * KROWB + pc * E * SZ) = kv4;
      const T* ve = reinterpret_cast<const T*>(&vv4);
      T* vcol = reinterpret_cast<T*>(vt) + key;
#pragma unroll
      for (int e = 0; e < E; ++e) vcol[(pc * E + e) * VROW] = ve[e];
    }
    __syncthreads();

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
    // online softmax for query r (log2 domain); keys 16mt + 4g + j
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 16 * mt + 4 * g + j;
        const float v = key < n_valid ? s[mt][j] * p.scale_log2 : -INFINITY;
        s[mt][j] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = exp2f(s[mt][j] - m_new);
        s[mt][j] = pv;
        l_run += pv;
      }
    m_run = m_new;

    // O^T += V^T P^T; contraction slots of lane group g hold the keys that
    // this lane's S^T registers hold
    if constexpr (SZ == 2) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        u32x4 bfrag;
        bfrag.x = f32_to_bf16(s[2 * cc][0]) | (f32_to_bf16(s[2 * cc][1]) << 16);
        bfrag.y = f32_to_bf16(s[2 * cc][2]) | (f32_to_bf16(s[2 * cc][3]) << 16);
        bfrag.z = f32_to_bf16(s[2 * cc + 1][0]) | (f32_to_bf16(s[2 * cc + 1][1]) << 16);
        bfrag.w = f32_to_bf16(s[2 * cc + 1][2]) | (f32_to_bf16(s[2 * cc + 1][3]) << 16);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const char* vrow = vt + (16 * dt + r) * VROWB;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + (32 * cc + 4 * g) * SZ);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + (32 * cc + 16 + 4 * g) * SZ);
          const u32x4 afrag = {lo.x, lo.y, hi.x, hi.y};
          mma16(o[dt], afrag, bfrag, T());
        }
      }
    } else {
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
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int64_t base = (((int64_t)b * p.Hq + hq) * p.nch + c) * p.K + r;
  float* po = p.part_o + base * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) po[16 * dt + 4 * g + j] = o[dt][j];
  if (g == 0) {
    p.part_ml[base * 2] = m_run;
    p.part_ml[base * 2 + 1] = l_tot;
  }
}

// o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the sequence's
// chunks (M = the largest m_c), in chunk order, written packed for the output
// projection.  One workgroup per (sequence, query head, 4 block queries);
// 32 lanes per query, each owning D/32 consecutive channels.
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs p) {
  constexpr int DPT = D / 32;
  const int groups = p.K / 4;
  const int bh = blockIdx.x / groups, qg = blockIdx.x % groups;
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int i = qg * 4 + (threadIdx.x >> 5);
  const int d0 = (threadIdx.x & 31) * DPT;
  int L = p.ctx_len[b];
  L = min(max(L, 0), p.max_len);
  const int nc = (L + p.K + p.chunk - 1) / p.chunk;
  const int64_t base = ((int64_t)b * p.Hq + hq) * p.nch * p.K + i;
  const float* ml = p.part_ml + base * 2;
  const int64_t cstride = (int64_t)p.K;  // entries between chunks
  float M = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < nc; ++c) M = fmaxf(M, ml[c * cstride * 2]);
  float ls = 0.f, acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll 8
  for (int c = 0; c < nc; ++c) {
    const float w = exp2f(ml[c * cstride * 2] - M);
    ls += w * ml[c * cstride * 2 + 1];
    const float* oc = p.part_o + (base + c * cstride) * D + d0;
#pragma unroll
    for (int k = 0; k < DPT; ++k) acc[k] += w * oc[k];
  }
  const float inv = 1.f / ls;
  const int row = b * p.K + i, Kd = p.Hq * D;
  T* dst = reinterpret_cast<T*>(static_cast<char*>(p.o) +
                                packed_offset<T>(row, hq * D + d0, Kd));
#pragma unroll
  for (int k = 0; k < DPT; ++k) store_elem(dst, k, acc[k] * inv);
}

template <typename T, int D>
hipError_t attn_t(int B, const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  hipLaunchKernelGGL((attn_partial_kernel<T, D>), dim3(a.nch, a.Hkv, B),
                     dim3(64 * G), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3(B * a.Hq * (a.K / 4)),
                     dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(bool bf16, int d, int B, const AttnArgs& a,
                            hipStream_t s) {
  if (d == 128) return bf16 ? attn_t<bf16_t, 128>(B, a, s) : attn_t<float, 128>(B, a, s);
  if (d == 64) return bf16 ? attn_t<bf16_t, 64>(B, a, s) : attn_t<float, 64>(B, a, s);
  return hipErrorInvalidValue;
}

}  // namespace dflash
