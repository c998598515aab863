// Internal launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace dflash {

constexpr int kMaxASeg = 8;
constexpr int kMaxBSeg = 16;

// C[M, N] = A[M, Kd] . B[N, Kd]^T, one grid-z slice of the contraction per
// partial.  A is split along the contraction into segments of a_seg_k
// elements (the concatenated target layers); B is split along N into
// segments with separate base pointers (e.g. Wq | Wk | Wv).
struct GemmArgs {
  const void* a_ptr[kMaxASeg];
  int64_t lda;       // row stride of every A segment, elements
  int a_seg_k;       // contraction width of each A segment
  const void* b_ptr[kMaxBSeg];
  int b_n0[kMaxBSeg + 1];  // segment s = output columns [b_n0[s], b_n0[s+1])
  int b_nseg;
  int M, N, Kd;
  int k_split;       // contraction elements per grid-z slice
  float* out;        // [gridDim.z][M][N] fp32 partial sums
};

struct GemmPlan {
  int MT;            // 16-row tiles per wave
  int gx, gy, gz;    // grid: column groups, row groups, contraction slices
  int k_split;
  size_t partial_floats;  // gz * M * N
};

constexpr int kGemmNT = 4;  // 16-column tiles per workgroup

GemmPlan plan_gemm(int M, int N, int Kd, bool bf16, int num_cu);
GemmPlan plan_lmhead(int M, int N, int Kd, bool bf16);
hipError_t launch_gemm(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                       hipStream_t s);
// LM head: full contraction per workgroup; per row and 64-column tile writes
// one Top2 record to part[row * gx + tile]; optional logits rows via rowmap.
hipError_t launch_lmhead(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                         Top2* part, float* logits, const int* rowmap,
                         int64_t logits_ld, hipStream_t s);

// ---- epilogues (epilogue.hip) ------------------------------------------
struct BlockState {
  int32_t* tokens;     // [B][K] current block ids
  int32_t* committed;  // [B][K] 1 = fixed
  int32_t* rowmap;     // [B * n_cap] compact LM-head row -> b*(K-1) + i-1
  int* err;
};

hipError_t launch_embed(bool bf16, int B, int K, int D, int V, int mask_id,
                        int pass, int n_cap, const int32_t* anchor,
                        const int32_t* block_tokens, BlockState st,
                        const void* embed, const void* gain, float eps,
                        float* x, void* h, void* hf, int32_t* draft,
                        hipStream_t s);

hipError_t launch_rows_rmsnorm(bool bf16, int rows, int D, int nsplit,
                               const float* part, const void* gain, float eps,
                               void* out, hipStream_t s);

hipError_t launch_kv_inject_epilogue(bool bf16, int T, int nlayers, int Hkv,
                                     int d, int nsplit, const float* part,
                                     const int32_t* row_seq,
                                     const int32_t* row_pos,
                                     const float2* rope, int max_batch,
                                     int max_ctx, int P, void* kv, int* err,
                                     hipStream_t s);

hipError_t launch_qkv_epilogue(bool bf16, int B, int K, int Hq, int Hkv, int d,
                               int nsplit, const float* part,
                               const int32_t* ctx_len, int max_len,
                               const float2* rope, int P, int max_batch,
                               void* q, void* kv_layer, int* err,
                               hipStream_t s);

// x += sum of partials; then either h = RMSNorm(x) * g (all rows) or, in
// final mode, compact still-masked rows into hf with the final gain.
hipError_t launch_resid_norm(bool bf16, int rows, int K, int D, int nsplit,
                             const float* part, float* x, const void* gain,
                             float eps, void* h, bool final_mode, int n_cap,
                             BlockState st, hipStream_t s);

hipError_t launch_swiglu(bool bf16, int rows, int I, int nsplit,
                         const float* part, void* act, hipStream_t s);

// ---- attention (attention.hip) -----------------------------------------
struct AttnArgs {
  const void* q;        // [B*K][Hq*d]
  const void* kc;       // this layer's K cache [max_batch][Hkv][P][d]
  const void* vc;       // this layer's V cache
  const int32_t* ctx_len;
  int max_len;          // host bound on ctx_len (grid sized for it)
  int P, Hq, Hkv, K;
  int chunk, nch;       // keys per workgroup, chunks per (sequence, kv head)
  float scale_log2;     // log2(e) / sqrt(d)
  float* part_o;        // [B][Hq][nch][K][d]
  float* part_ml;       // [B][Hq][nch][K][2]
  void* o;              // [B*K][Hq*d]
};
hipError_t launch_attention(bool bf16, int d, int B, const AttnArgs& a,
                            hipStream_t s);

// ---- head (head.hip) -----------------------------------------------------
struct RowResult {
  int32_t token;
  float conf;
  float margin;
  float lse;
};
hipError_t launch_lm_merge(int rows, int ntiles, const Top2* part,
                           RowResult* res, hipStream_t s);
hipError_t launch_commit(int B, int K, int n_cap, int commit, bool last,
                         const RowResult* res, BlockState st,
                         int32_t* draft, float* conf, float* margin,
                         hipStream_t s);
hipError_t launch_verify(int B, int K, const int32_t* draft,
                         const int32_t* target, int32_t* accept,
                         int32_t* next_anchor, hipStream_t s);

}  // namespace dflash
