// Row kernels: the block embedding at the start of each drafting pass
// (x = E[token] into the fp32 residual rows) and RMSNorm of residual rows
// into the packed operand layout that the next GEMM reads.
//
// Pass 0 also sets up the block: [anchor, mask, ..., mask] or the caller's
// block, with index 0 and non-mask ids committed.  Every pass rebuilds the
// map from LM-head rows to still-masked block rows (rank by block index).
#include <algorithm>

#include "../../include/dflash.h"
#include "kernels.h"

namespace dflash {

namespace {

__device__ __forceinline__ bool masked_at(int pass, int b, int i, int K,
                                          int mask_id,
                                          const int32_t* block_tokens,
                                          const int32_t* committed) {
  if (i == 0) return false;
  if (pass > 0) return committed[b * K + i] == 0;
  return block_tokens == nullptr || block_tokens[b * K + i] == mask_id;
}

// One workgroup per block row.  Wave 0 sets up the row (pass 0: token from
// the anchor / caller block, validated; committed flag; caller-committed ids
// into the draft) and, in the workgroup of a sequence's index 0, the LM-head
// row map (lane j = block index j; rank among masked positions by ballot).
// Then x[row] = E[token] in fp32.  With a gain g0 the workgroup also writes
// RMSNorm(x[row]) * g0 packed into h0 (the first layer's input; statistics
// in float64, one rounding), which saves a separate pass over x.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(
    int K, int D, int V, int mask_id, int pass, int n_cap,
    const int32_t* anchor, const int32_t* block_tokens, BlockState st,
    const T* E, float* x, int32_t* draft, const T* g0, float eps, T* h0) {
  constexpr int EL = Storage<T>::E;
  __shared__ int tok_s;
  __shared__ double red_s[4];
  const int row = blockIdx.x, b = row / K, i = row % K;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    if (lane == 0) {
      int tok;
      if (pass == 0) {
        tok = block_tokens != nullptr ? block_tokens[row]
                                      : (i == 0 ? anchor[b] : mask_id);
        const int com = !masked_at(0, b, i, K, mask_id, block_tokens, nullptr);
        if (tok < 0 || tok >= V) {
          set_error(st.err, DFLASH_DEVERR_TOKEN);
          tok = min(max(tok, 0), V - 1);
        }
        st.tokens[row] = tok;
        st.committed[row] = com;
        // a caller-committed position is part of the returned draft as given
        if (com && i > 0) draft[b * (K - 1) + i - 1] = tok;
      } else {
        tok = st.tokens[row];
        if (tok < 0 || tok >= V) {  // a commit that found no finite logit
          set_error(st.err, DFLASH_DEVERR_TOKEN);
          tok = min(max(tok, 0), V - 1);
        }
      }
      tok_s = tok;
    }
    if (i == 0) {
      // LM-head rows of this sequence: still-masked positions by index
      const bool m = lane > 0 && lane < K &&
                     masked_at(pass, b, lane, K, mask_id, block_tokens,
                               st.committed);
      const unsigned long long ball = __ballot(m);
      const int rank = __popcll(ball & ((1ull << lane) - 1ull));
      if (m && rank < n_cap) st.rowmap[b * n_cap + rank] = b * K + lane;
      const int count = min(__popcll(ball), n_cap);
      if (lane >= count && lane < n_cap) st.rowmap[b * n_cap + lane] = -1;
    }
  }
  __syncthreads();
  const int tok = tok_s;
  const char* src = reinterpret_cast<const char*>(E + (int64_t)tok * D);
  float* xr = x + (int64_t)row * D;
  const int nch = D / EL;
  double ss = 0.0;
  for (int c = threadIdx.x; c < nch; c += 256) {
    const u32x4 v = load16(src + (int64_t)c * 16);
    const T* vt = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int e = 0; e < EL; e += 4) {
      const f32x4 f = {load_elem(vt, e), load_elem(vt, e + 1),
                       load_elem(vt, e + 2), load_elem(vt, e + 3)};
      *reinterpret_cast<f32x4*>(xr + c * EL + e) = f;
      ss += (double)f.x * f.x + (double)f.y * f.y + (double)f.z * f.z +
            (double)f.w * f.w;
    }
  }
  if (g0 == nullptr) return;
  const double inv = 1.0 / sqrt(block_sum<4>(ss, red_s) / (double)D + (double)eps);
  char* ob = reinterpret_cast<char*>(h0);
  for (int c = threadIdx.x; c < nch; c += 256) {
    const u32x4 v = load16(src + (int64_t)c * 16);  // cached: just read
    const u32x4 gv = load16(g0 + c * EL);
    const T* vt = reinterpret_cast<const T*>(&v);
    const T* gt = reinterpret_cast<const T*>(&gv);
    u32x4 o;  // the 16-byte chunk is built in registers, stored once
    T* ot = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int e = 0; e < EL; ++e)
      store_elem(ot, e, (double)load_elem(vt, e) * inv * (double)load_elem(gt, e));
    *reinterpret_cast<u32x4*>(ob + packed_offset<T>(row, c * EL, D)) = o;
  }
}

// out[row] = RMSNorm(x[src]) * g written packed (statistics and scaling in
// float64, one rounding to the storage type), src = rowmap ? rowmap[row]
// : row; rows without a source (padding to a multiple of 16, unmapped LM-head
// rows) are written as zeros.  One workgroup per row, one thread per 16-byte
// chunk: the fastest form up to a few hundred rows.
constexpr int kNormChunks = 4;  // chunks per thread: D <= 256 * E * 4
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_row_kernel(int rows, int D,
                                                          const float* x,
                                                          const int32_t* rowmap,
                                                          const T* g, float eps,
                                                          T* out) {
  constexpr int E = Storage<T>::E;
  __shared__ double scratch[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int src = row < rows ? (rowmap ? rowmap[row] : row) : -1;
  char* ob = reinterpret_cast<char*>(out);
  const int nch = D / E;
  if (src < 0) {
    for (int c = tid; c < nch; c += 256)
      *reinterpret_cast<u32x4*>(ob + packed_offset<T>(row, c * E, D)) =
          u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const float* xr = x + (int64_t)src * D;
  float v[kNormChunks][E];
  double ss = 0.0;
#pragma unroll
  for (int ci = 0; ci < kNormChunks; ++ci) {
    const int c = tid + ci * 256;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        const f32x4 q = __builtin_bit_cast(f32x4, load16(xr + c * E + e));
        v[ci][e] = q.x;
        v[ci][e + 1] = q.y;
        v[ci][e + 2] = q.z;
        v[ci][e + 3] = q.w;
        ss += (double)q.x * q.x + (double)q.y * q.y + (double)q.z * q.z +
              (double)q.w * q.w;
      }
    }
  }
  const double tot = block_sum<4>(ss, scratch);
  const double inv = 1.0 / sqrt(tot / (double)D + (double)eps);
#pragma unroll
  for (int ci = 0; ci < kNormChunks; ++ci) {
    const int c = tid + ci * 256;
    if (c < nch) {
      const u32x4 gv = load16(g + c * E);
      const T* gt = reinterpret_cast<const T*>(&gv);
      u32x4 o;  // the 16-byte chunk is built in registers, stored once
      T* ot = reinterpret_cast<T*>(&o);
#pragma unroll
      for (int e = 0; e < E; ++e)
        store_elem(ot, e, (double)v[ci][e] * inv * (double)load_elem(gt, e));
      *reinterpret_cast<u32x4*>(ob + packed_offset<T>(row, c * E, D)) = o;
    }
  }
}

// A split-K reduction fused with the row RMSNorm that reads its result: for
// row r < M, x[r] = sum_s ws[s][r] (plus the old x[r] when resid), the
// copies added in order in float exactly as splitk_reduce_kernel adds them,
// is written back,
// and out[r] = RMSNorm(x[r]) * g is written packed with rmsnorm_row_kernel's
// arithmetic (the same chunks per thread, the same float64 sums and
// rounding).  So x and out are bit for bit those of the two kernels run one
// after the other, with one launch and one pass over x fewer.  Rows from M
// to the next multiple of 16 are written as zeros.
// The number of copies S is a template argument so that every load of a
// thread (S copies and the old x of each of its chunks) is issued before the
// first is used: one memory latency per row instead of one per copy.
template <typename T, int S>
__global__ __launch_bounds__(256) void splitk_norm_row_kernel(
    int M, int D, const float* ws, float* x, int resid, const T* g,
    float eps, T* out) {
  constexpr int E = Storage<T>::E, E4 = E / 4;
  __shared__ double scratch[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  char* ob = reinterpret_cast<char*>(out);
  const int nch = D / E;
  if (row >= M) {
    for (int c = tid; c < nch; c += 256)
      *reinterpret_cast<u32x4*>(ob + packed_offset<T>(row, c * E, D)) =
          u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const int64_t plane = (int64_t)M * D;
  float* xr = x + (int64_t)row * D;
  const float* wr = ws + (int64_t)row * D;
  f32x4 w[kNormChunks][E4][S], o[kNormChunks][E4];
#pragma unroll
  for (int ci = 0; ci < kNormChunks; ++ci) {
    const int c = tid + ci * 256;
    if (c < nch) {
#pragma unroll
      for (int e4 = 0; e4 < E4; ++e4) {
        const int col = c * E + 4 * e4;
#pragma unroll
        for (int k = 0; k < S; ++k)
          w[ci][e4][k] =
              *reinterpret_cast<const f32x4*>(wr + k * plane + col);
        if (resid) o[ci][e4] = *reinterpret_cast<const f32x4*>(xr + col);
      }
    }
  }
  float v[kNormChunks][E];
  double ss = 0.0;
#pragma unroll
  for (int ci = 0; ci < kNormChunks; ++ci) {
    const int c = tid + ci * 256;
    if (c < nch) {
#pragma unroll
      for (int e4 = 0; e4 < E4; ++e4) {
        const int col = c * E + 4 * e4;
        f32x4 q = w[ci][e4][0];
#pragma unroll
        for (int k = 1; k < S; ++k)
          q = f32x4{q[0] + w[ci][e4][k][0], q[1] + w[ci][e4][k][1],
                    q[2] + w[ci][e4][k][2], q[3] + w[ci][e4][k][3]};
        if (resid) {
          const f32x4 a = o[ci][e4];
          q = f32x4{a[0] + q[0], a[1] + q[1], a[2] + q[2], a[3] + q[3]};
        }
        *reinterpret_cast<f32x4*>(xr + col) = q;
        const int e = 4 * e4;
        v[ci][e] = q.x;
        v[ci][e + 1] = q.y;
        v[ci][e + 2] = q.z;
        v[ci][e + 3] = q.w;
        ss += (double)q.x * q.x + (double)q.y * q.y + (double)q.z * q.z +
              (double)q.w * q.w;
      }
    }
  }
  const double tot = block_sum<4>(ss, scratch);
  const double inv = 1.0 / sqrt(tot / (double)D + (double)eps);
#pragma unroll
  for (int ci = 0; ci < kNormChunks; ++ci) {
    const int c = tid + ci * 256;
    if (c < nch) {
      const u32x4 gv = load16(g + c * E);
      const T* gt = reinterpret_cast<const T*>(&gv);
      u32x4 ov;  // the 16-byte chunk is built in registers, stored once
      T* ot = reinterpret_cast<T*>(&ov);
#pragma unroll
      for (int e = 0; e < E; ++e)
        store_elem(ot, e, (double)v[ci][e] * inv * (double)load_elem(gt, e));
      *reinterpret_cast<u32x4*>(ob + packed_offset<T>(row, c * E, D)) = ov;
    }
  }
}

// The same, one workgroup per 16-row tile of the packed output, wave r on
// row r (faster from ~512 rows, where the row form's partial-fragment
// stores dominate).
// First each wave reduces its row's sum of squares (the row map picks the
// source row; -1 and rows past `rows` give a zero row); then every wave
// writes whole 1 KiB fragments of the packed tile (lane l: tile row l % 16,
// contraction group l / 16), so every store is part of one contiguous
// wave-wide write.
// The tile's contraction steps are split over gridDim.y workgroups (each
// recomputes the 16 rows' statistics, from L2), so that a few hundred rows
// still fill the chip.
template <typename T>
__global__ __launch_bounds__(1024) void rmsnorm_tile_kernel(int rows, int D,
                                                       const float* x,
                                                       const int32_t* rowmap,
                                                       const T* g, float eps,
                                                       T* out) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC;
  __shared__ double inv_s[16];
  __shared__ int src_s[16];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = blockIdx.y, nparts = gridDim.y;
  {
    const int row = t * 16 + wave;
    const int src = row < rows ? (rowmap ? rowmap[row] : row) : -1;
    double ss = 0.0;
    if (src >= 0) {
      const float* xr = x + (int64_t)src * D;
#pragma unroll 8
      for (int c = lane * 4; c < D; c += 256) {
        const f32x4 q = __builtin_bit_cast(f32x4, load16(xr + c));
        ss += (double)q.x * q.x + (double)q.y * q.y + (double)q.z * q.z +
              (double)q.w * q.w;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) {
      inv_s[wave] = 1.0 / sqrt(ss / (double)D + (double)eps);
      src_s[wave] = src;
    }
  }
  __syncthreads();
  const int r = lane & 15, grp = lane >> 4;
  const int src = src_s[r];
  const double inv = inv_s[r];
  const int nsteps = D / KC;
  // this workgroup's steps [s_lo, s_hi)
  const int s_lo = (int)((int64_t)part * nsteps / nparts);
  const int s_hi = (int)((int64_t)(part + 1) * nsteps / nparts);
  char* ob = reinterpret_cast<char*>(out) + ((int64_t)t * nsteps * 64 + lane) * 16;
  if (src < 0) {  // lanes of rows without a source write zeros
    for (int s = s_lo + wave; s < s_hi; s += 16)
      *reinterpret_cast<u32x4*>(ob + (int64_t)s * 1024) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const float* xr = x + (int64_t)src * D + grp * E;
  const T* gk = g + grp * E;
  constexpr int U = 4;  // fragments whose loads are in flight together
  for (int s0 = s_lo + wave; s0 < s_hi; s0 += 16 * U) {
    u32x4 gv[U], q[U][E / 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + 16 * u, s_hi - 1);
      gv[u] = load16(gk + s * KC);
#pragma unroll
      for (int e = 0; e < E / 4; ++e) q[u][e] = load16(xr + s * KC + 4 * e);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 16 * u;
      if (s >= s_hi) break;
      const T* gt = reinterpret_cast<const T*>(&gv[u]);
      u32x4 v;
      T* vt = reinterpret_cast<T*>(&v);
#pragma unroll
      for (int e = 0; e < E; ++e)
        store_elem(vt, e,
                   (double)__builtin_bit_cast(f32x4, q[u][e / 4])[e % 4] * inv *
                       (double)load_elem(gt, e));
      *reinterpret_cast<u32x4*>(ob + (int64_t)s * 1024) = v;
    }
  }
}

template <typename T>
hipError_t embed_t(int B, int K, int D, int V, int mask_id, int pass,
                   int n_cap, const int32_t* anchor, const int32_t* block_tokens,
                   BlockState st, const void* embed, float* x,
                   int32_t* draft, const void* g0, float eps, void* h0,
                   hipStream_t s) {
  launch_k(embed_kernel<T>, dim3(B * K), dim3(256), 0, s, K, D, V,
                     mask_id, pass, n_cap, anchor, block_tokens, st,
                     static_cast<const T*>(embed), x, draft,
                     static_cast<const T*>(g0), eps, static_cast<T*>(h0));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_embed(bool bf16, int B, int K, int D, int V, int mask_id,
                        int pass, int n_cap, const int32_t* anchor,
                        const int32_t* block_tokens, BlockState st,
                        const void* embed, float* x, int32_t* draft,
                        const void* g0, float eps, void* h0, hipStream_t s) {
  return bf16 ? embed_t<bf16_t>(B, K, D, V, mask_id, pass, n_cap, anchor,
                                block_tokens, st, embed, x, draft, g0, eps, h0,
                                s)
              : embed_t<float>(B, K, D, V, mask_id, pass, n_cap, anchor,
                               block_tokens, st, embed, x, draft, g0, eps, h0,
                               s);
}

bool rmsnorm_row_form(bool bf16, int rows, int D) {
  return (rows + 15) / 16 < 32 && D <= 256 * kNormChunks * (bf16 ? 8 : 4);
}

template <int S>
hipError_t splitk_norm_t(bool bf16, int tiles, int M, int D, const float* ws,
                         float* x, bool resid, const void* gain, float eps,
                         void* out, hipStream_t s) {
  if (bf16)
    launch_k(splitk_norm_row_kernel<bf16_t, S>, dim3(tiles * 16), dim3(256),
             0, s, M, D, ws, x, resid ? 1 : 0,
             static_cast<const bf16_t*>(gain), eps, static_cast<bf16_t*>(out));
  else
    launch_k(splitk_norm_row_kernel<float, S>, dim3(tiles * 16), dim3(256), 0,
             s, M, D, ws, x, resid ? 1 : 0, static_cast<const float*>(gain),
             eps, static_cast<float*>(out));
  return hipGetLastError();
}

// S = 1 to 4 copies (the most a split GEMM makes)
hipError_t launch_splitk_norm(bool bf16, int M, int D, int S, const float* ws,
                              float* x, bool resid, const void* gain,
                              float eps, void* out, hipStream_t s) {
  if (!rmsnorm_row_form(bf16, M, D) || S < 1 || M < 1 ||
      D % (bf16 ? 8 : 4) != 0)
    return hipErrorInvalidValue;
  const int tiles = (M + 15) / 16;
  switch (S) {
    case 1: return splitk_norm_t<1>(bf16, tiles, M, D, ws, x, resid, gain, eps, out, s);
    case 2: return splitk_norm_t<2>(bf16, tiles, M, D, ws, x, resid, gain, eps, out, s);
    case 3: return splitk_norm_t<3>(bf16, tiles, M, D, ws, x, resid, gain, eps, out, s);
    case 4: return splitk_norm_t<4>(bf16, tiles, M, D, ws, x, resid, gain, eps, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rmsnorm(bool bf16, int rows, int D, const float* x,
                          const int32_t* rowmap, const void* gain, float eps,
                          void* out, hipStream_t s) {
  const int tiles = (rows + 15) / 16;
  if (rmsnorm_row_form(bf16, rows, D)) {
    if (bf16)
      launch_k(rmsnorm_row_kernel<bf16_t>, dim3(tiles * 16), dim3(256),
                         0, s, rows, D, x, rowmap,
                         static_cast<const bf16_t*>(gain), eps,
                         static_cast<bf16_t*>(out));
    else
      launch_k(rmsnorm_row_kernel<float>, dim3(tiles * 16), dim3(256),
                         0, s, rows, D, x, rowmap,
                         static_cast<const float*>(gain), eps,
                         static_cast<float*>(out));
    return hipGetLastError();
  }
  // about 256 workgroups, each with at least 16 contraction steps
  const int nsteps = D / (bf16 ? Storage<bf16_t>::KC : Storage<float>::KC);
  const int parts = std::max(1, std::min((256 + tiles - 1) / tiles,
                                         nsteps / 16));
  if (bf16)
    launch_k(rmsnorm_tile_kernel<bf16_t>, dim3(tiles, parts), dim3(1024), 0,
                       s, rows, D, x, rowmap, static_cast<const bf16_t*>(gain),
                       eps, static_cast<bf16_t*>(out));
  else
    launch_k(rmsnorm_tile_kernel<float>, dim3(tiles, parts), dim3(1024), 0,
                       s, rows, D, x, rowmap, static_cast<const float*>(gain),
                       eps, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace dflash
