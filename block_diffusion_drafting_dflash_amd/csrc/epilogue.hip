// Row-wise kernels around the GEMMs: block embedding, summing the split-K
// partials, RMSNorm, RoPE, SwiGLU, and the scatter of K/V into the cache.
//
// Each row kernel runs one 256-thread workgroup per row; partial slices are
// summed in slice order and norms reduce in a fixed tree, so results do not
// depend on scheduling.
#include "../../include/dflash.h"
#include "kernels.h"

namespace dflash {

namespace {

// Sum of the split-K slices of partial element (row, col).
__device__ __forceinline__ float sum_slices(const float* part, int nsplit,
                                            int rows, int N, int row, int col) {
  float v = 0.f;
  for (int z = 0; z < nsplit; ++z)
    v += part[((int64_t)z * rows + row) * N + col];
  return v;
}

// Block: tokens [anchor, mask, ...] (or the caller's block), x = E[token],
// h = RMSNorm(x) * g of the first layer.  Pass 0 also initialises the
// block state; every pass resets the compact-row map.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(
    int K, int D, int V, int mask_id, int pass, int n_cap,
    const int32_t* anchor, const int32_t* block_tokens, BlockState st,
    const T* E, const T* g, float eps, float* x, T* h, T* hf, int32_t* draft) {
  __shared__ float scratch[4];
  __shared__ int tok_s;
  const int row = blockIdx.x, b = row / K, i = row % K;
  if (threadIdx.x == 0) {
    if (pass == 0) {
      int tok, com;
      if (block_tokens != nullptr) {
        tok = block_tokens[row];
        com = (i == 0) || (tok != mask_id);
      } else {
        tok = (i == 0) ? anchor[b] : mask_id;
        com = (i == 0);
      }
      if (tok < 0 || tok >= V) {
        set_error(st.err, DFLASH_DEVERR_TOKEN);
        tok = min(max(tok, 0), V - 1);
      }
      st.tokens[row] = tok;
      st.committed[row] = com;
      // a caller-committed position is part of the returned draft as given
      if (com && i > 0) draft[b * (K - 1) + i - 1] = tok;
    }
    tok_s = st.tokens[row];
    if (i < n_cap) st.rowmap[b * n_cap + i] = -1;
  }
  // a caller-given block may leave compact LM-head rows unused: zero them
  if (block_tokens != nullptr && i < n_cap) {
    T* dst = hf + (int64_t)(b * n_cap + i) * D;
    for (int c = threadIdx.x; c < D; c += 256) store_elem(dst, c, 0.f);
  }
  __syncthreads();
  const int tok = tok_s;
  const T* src = E + (int64_t)tok * D;
  float* xr = x + (int64_t)row * D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float v = load_elem(src, c);
    xr[c] = v;
    ss += v * v;
  }
  const float tot = block_sum<4>(ss, scratch);
  const float inv = 1.f / sqrtf(tot / (float)D + eps);
  T* hr = h + (int64_t)row * D;
  for (int c = threadIdx.x; c < D; c += 256)
    store_elem(hr, c, xr[c] * inv * load_elem(g, c));
}

// out = RMSNorm(sum of slices) * g  (fused target features H_cond)
template <typename T>
__global__ __launch_bounds__(256) void rows_rmsnorm_kernel(
    int rows, int D, int nsplit, const float* part, const T* g, float eps,
    T* out) {
  extern __shared__ float u[];
  __shared__ float scratch[4];
  const int row = blockIdx.x;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float v = sum_slices(part, nsplit, rows, D, row, c);
    u[c] = v;
    ss += v * v;
  }
  const float tot = block_sum<4>(ss, scratch);
  const float inv = 1.f / sqrtf(tot / (float)D + eps);
  T* o = out + (int64_t)row * D;
  for (int c = threadIdx.x; c < D; c += 256)
    store_elem(o, c, u[c] * inv * load_elem(g, c));
}

// Injected rows: K = RoPE(sum), V = sum, written to every layer's cache.
// Columns of the fused projection: layer l occupies [l*2*Hkv*d, (l+1)*...),
// its K heads first, then its V heads.
template <typename T>
__global__ __launch_bounds__(256) void kv_inject_epilogue_kernel(
    int rows, int nlayers, int Hkv, int d, int nsplit, const float* part,
    const int32_t* row_seq, const int32_t* row_pos, const float2* rope,
    int max_batch, int max_ctx, int P, T* kv, int* err) {
  const int row = blockIdx.x;
  const int seq = row_seq[row], pos = row_pos[row];
  if (seq < 0 || seq >= max_batch) {
    if (threadIdx.x == 0) set_error(err, DFLASH_DEVERR_SLOT);
    return;
  }
  if (pos < 0 || pos >= max_ctx) {
    if (threadIdx.x == 0) set_error(err, DFLASH_DEVERR_POS);
    return;
  }
  const int half = d / 2, kvd = Hkv * d, N = nlayers * 2 * kvd;
  const int64_t layer_stride = (int64_t)2 * max_batch * Hkv * P * d;
  const int64_t kv_stride = (int64_t)max_batch * Hkv * P * d;
  const int work = nlayers * Hkv * half;
  for (int w = threadIdx.x; w < work; w += 256) {
    const int l = w / (Hkv * half), rem = w % (Hkv * half);
    const int hh = rem / half, i = rem % half;
    const int cb = l * 2 * kvd + hh * d;
    const float k0 = sum_slices(part, nsplit, rows, N, row, cb + i);
    const float k1 = sum_slices(part, nsplit, rows, N, row, cb + i + half);
    const float v0 = sum_slices(part, nsplit, rows, N, row, cb + kvd + i);
    const float v1 = sum_slices(part, nsplit, rows, N, row, cb + kvd + i + half);
    const float2 cs = rope[(int64_t)pos * half + i];
    T* kd = kv + l * layer_stride + (((int64_t)seq * Hkv + hh) * P + pos) * d;
    T* vd = kd + kv_stride;
    store_elem(kd, i, k0 * cs.x - k1 * cs.y);
    store_elem(kd, i + half, k1 * cs.x + k0 * cs.y);
    store_elem(vd, i, v0);
    store_elem(vd, i + half, v1);
  }
}

// Block rows after the QKV projection: q = RoPE(q) -> q buffer; the block's
// own k = RoPE(k), v -> cache positions L_b + i (scratch for this draft).
template <typename T>
__global__ __launch_bounds__(256) void qkv_epilogue_kernel(
    int K, int Hq, int Hkv, int d, int nsplit, int rows, const float* part,
    const int32_t* ctx_len, int max_len, const float2* rope, int P,
    int max_batch, T* q, T* kv_layer, int* err) {
  const int row = blockIdx.x, b = row / K, i = row % K;
  int L = ctx_len[b];
  if (L < 0 || L > max_len) {  // attention clamps the same way
    if (threadIdx.x == 0) set_error(err, DFLASH_DEVERR_CTX_LEN);
    L = min(max(L, 0), max_len);
  }
  const int pos = L + i;
  const int half = d / 2, qd = Hq * d, kvd = Hkv * d, N = qd + 2 * kvd;
  T* kc = kv_layer;
  T* vc = kv_layer + (int64_t)max_batch * Hkv * P * d;
  const float2* cs_row = rope + (int64_t)pos * half;
  for (int w = threadIdx.x; w < (Hq + Hkv) * half; w += 256) {
    const int hh = w / half, j = w % half;
    const int cb = hh * d;  // q heads then k heads are contiguous columns
    const float a0 = sum_slices(part, nsplit, rows, N, row, cb + j);
    const float a1 = sum_slices(part, nsplit, rows, N, row, cb + j + half);
    const float2 cs = cs_row[j];
    const float r0 = a0 * cs.x - a1 * cs.y, r1 = a1 * cs.x + a0 * cs.y;
    if (hh < Hq) {
      T* dst = q + (int64_t)row * qd + cb;
      store_elem(dst, j, r0);
      store_elem(dst, j + half, r1);
    } else {
      const int kh = hh - Hq;
      T* dst = kc + (((int64_t)b * Hkv + kh) * P + pos) * d;
      store_elem(dst, j, r0);
      store_elem(dst, j + half, r1);
    }
  }
  for (int w = threadIdx.x; w < kvd; w += 256) {
    const int kh = w / d, e = w % d;
    const float v = sum_slices(part, nsplit, rows, N, row, qd + kvd + w);
    store_elem(vc + (((int64_t)b * Hkv + kh) * P + pos) * d, e, v);
  }
}

// x += sum of slices; then h = RMSNorm(x) * g for every row, or (final
// mode) only for still-masked rows, compacted per sequence into hf with the
// LM-head row map.
template <typename T>
__global__ __launch_bounds__(256) void resid_norm_kernel(
    int rows, int K, int D, int nsplit, const float* part, float* x,
    const T* g, float eps, T* h, int final_mode, int n_cap, BlockState st) {
  __shared__ float scratch[4];
  __shared__ int dst_row;
  const int row = blockIdx.x;
  if (final_mode) {
    if (threadIdx.x == 0) {
      const int b = row / K, i = row % K;
      int dr = -1;
      if (!st.committed[row]) {
        int rank = 0;
        for (int j = 0; j < i; ++j) rank += st.committed[b * K + j] ? 0 : 1;
        dr = b * n_cap + rank;
        st.rowmap[dr] = b * (K - 1) + (i - 1);
      }
      dst_row = dr;
    }
    __syncthreads();
    if (dst_row < 0) return;
  }
  float* xr = x + (int64_t)row * D;
  float ss = 0.f;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float v = xr[c] + sum_slices(part, nsplit, rows, D, row, c);
    xr[c] = v;
    ss += v * v;
  }
  const float tot = block_sum<4>(ss, scratch);
  const float inv = 1.f / sqrtf(tot / (float)D + eps);
  T* hr = h + (int64_t)(final_mode ? dst_row : row) * D;
  for (int c = threadIdx.x; c < D; c += 256)
    store_elem(hr, c, xr[c] * inv * load_elem(g, c));
}

// act = silu(gate) * up; columns [0, I) gate, [I, 2I) up.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(int rows, int I,
                                                     int nsplit,
                                                     const float* part,
                                                     T* act) {
  const int64_t total = (int64_t)rows * I;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int r = (int)(idx / I), n = (int)(idx % I);
    const float gs = sum_slices(part, nsplit, rows, 2 * I, r, n);
    const float us = sum_slices(part, nsplit, rows, 2 * I, r, I + n);
    store_elem(act, idx, gs / (1.f + __expf(-gs)) * us);
  }
}

template <typename T> const T* cT(const void* p) { return static_cast<const T*>(p); }
template <typename T> T* mT(void* p) { return static_cast<T*>(p); }

template <typename T>
hipError_t embed_t(int B, int K, int D, int V, int mask_id, int pass,
                   int n_cap, const int32_t* anchor, const int32_t* block_tokens,
                   BlockState st, const void* embed, const void* gain, float eps,
                   float* x, void* h, void* hf, int32_t* draft, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel<T>, dim3(B * K), dim3(256), 0, s, K, D, V,
                     mask_id, pass, n_cap, anchor, block_tokens, st,
                     cT<T>(embed), cT<T>(gain), eps, x, mT<T>(h), mT<T>(hf),
                     draft);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_embed(bool bf16, int B, int K, int D, int V, int mask_id,
                        int pass, int n_cap, const int32_t* anchor,
                        const int32_t* block_tokens, BlockState st,
                        const void* embed, const void* gain, float eps,
                        float* x, void* h, void* hf, int32_t* draft,
                        hipStream_t s) {
  return bf16 ? embed_t<bf16_t>(B, K, D, V, mask_id, pass, n_cap, anchor,
                                block_tokens, st, embed, gain, eps, x, h, hf,
                                draft, s)
              : embed_t<float>(B, K, D, V, mask_id, pass, n_cap, anchor,
                               block_tokens, st, embed, gain, eps, x, h, hf,
                               draft, s);
}

hipError_t launch_rows_rmsnorm(bool bf16, int rows, int D, int nsplit,
                               const float* part, const void* gain, float eps,
                               void* out, hipStream_t s) {
  const size_t lds = (size_t)D * sizeof(float);
  if (bf16)
    hipLaunchKernelGGL(rows_rmsnorm_kernel<bf16_t>, dim3(rows), dim3(256), lds,
                       s, rows, D, nsplit, part, cT<bf16_t>(gain), eps,
                       mT<bf16_t>(out));
  else
    hipLaunchKernelGGL(rows_rmsnorm_kernel<float>, dim3(rows), dim3(256), lds,
                       s, rows, D, nsplit, part, cT<float>(gain), eps,
                       mT<float>(out));
  return hipGetLastError();
}

hipError_t launch_kv_inject_epilogue(bool bf16, int T, int nlayers, int Hkv,
                                     int d, int nsplit, const float* part,
                                     const int32_t* row_seq,
                                     const int32_t* row_pos,
                                     const float2* rope, int max_batch,
                                     int max_ctx, int P, void* kv, int* err,
                                     hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(kv_inject_epilogue_kernel<bf16_t>, dim3(T), dim3(256), 0,
                       s, T, nlayers, Hkv, d, nsplit, part, row_seq, row_pos,
                       rope, max_batch, max_ctx, P, mT<bf16_t>(kv), err);
  else
    hipLaunchKernelGGL(kv_inject_epilogue_kernel<float>, dim3(T), dim3(256), 0,
                       s, T, nlayers, Hkv, d, nsplit, part, row_seq, row_pos,
                       rope, max_batch, max_ctx, P, mT<float>(kv), err);
  return hipGetLastError();
}

hipError_t launch_qkv_epilogue(bool bf16, int B, int K, int Hq, int Hkv, int d,
                               int nsplit, const float* part,
                               const int32_t* ctx_len, int max_len,
                               const float2* rope, int P, int max_batch,
                               void* q, void* kv_layer, int* err,
                               hipStream_t s) {
  const int rows = B * K;
  if (bf16)
    hipLaunchKernelGGL(qkv_epilogue_kernel<bf16_t>, dim3(rows), dim3(256), 0, s,
                       K, Hq, Hkv, d, nsplit, rows, part, ctx_len, max_len,
                       rope, P, max_batch, mT<bf16_t>(q), mT<bf16_t>(kv_layer),
                       err);
  else
    hipLaunchKernelGGL(qkv_epilogue_kernel<float>, dim3(rows), dim3(256), 0, s,
                       K, Hq, Hkv, d, nsplit, rows, part, ctx_len, max_len,
                       rope, P, max_batch, mT<float>(q), mT<float>(kv_layer),
                       err);
  return hipGetLastError();
}

hipError_t launch_resid_norm(bool bf16, int rows, int K, int D, int nsplit,
                             const float* part, float* x, const void* gain,
                             float eps, void* h, bool final_mode, int n_cap,
                             BlockState st, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(resid_norm_kernel<bf16_t>, dim3(rows), dim3(256), 0, s,
                       rows, K, D, nsplit, part, x, cT<bf16_t>(gain), eps,
                       mT<bf16_t>(h), final_mode ? 1 : 0, n_cap, st);
  else
    hipLaunchKernelGGL(resid_norm_kernel<float>, dim3(rows), dim3(256), 0, s,
                       rows, K, D, nsplit, part, x, cT<float>(gain), eps,
                       mT<float>(h), final_mode ? 1 : 0, n_cap, st);
  return hipGetLastError();
}

hipError_t launch_swiglu(bool bf16, int rows, int I, int nsplit,
                         const float* part, void* act, hipStream_t s) {
  const int64_t total = (int64_t)rows * I;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(swiglu_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s,
                       rows, I, nsplit, part, mT<bf16_t>(act));
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       rows, I, nsplit, part, mT<float>(act));
  return hipGetLastError();
}

}  // namespace dflash
