// Internal launch interface between the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"
#include "common.h"

namespace dflash {

// Benchmark timing of one kernel class.  While a pair of events is armed,
// every launch made through launch_k binds them to its own dispatch: the
// first launch of the span takes the start event, each launch takes the stop
// event (the last one wins), so the pair brackets the class's kernels without
// any event packet of its own entering the stream.
struct DispatchTiming {
  hipEvent_t start = nullptr;  // taken by the next launch
  hipEvent_t stop = nullptr;   // taken by the last of `kernels` launches
  int kernels = 1;
};
DispatchTiming& dispatch_timing();  // per host thread

template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, uint32_t shm,
                     hipStream_t s, Args... args) {
  DispatchTiming& t = dispatch_timing();
  hipExtLaunchKernelGGL(kernel, grid, block, shm, s, t.start,
                        t.kernels <= 1 ? t.stop : nullptr, 0u, args...);
  t.start = nullptr;
  if (t.kernels > 1) --t.kernels;
}

constexpr int kMaxASeg = 8;
constexpr int kMaxBSeg = 16;

// ---------------------------------------------------------------------------
// Fragment-major ("packed") operands.
//
// An MFMA fragment is 16 rows x KC contraction elements, 16 bytes per lane:
// lane l holds row l % 16, elements [(l / 16) * E, +E) of the step.  A packed
// matrix with R rows (R % 16 == 0) and contraction K stores fragment
// (row tile t, step s) as 1 KiB at byte ((t * (K / KC) + s) * 64 + l) * 16, so
// every wave-wide operand load is one contiguous 1 KiB.  Weights are packed
// once at create time, activations are written packed by the kernel that
// produces them.
// ---------------------------------------------------------------------------
template <typename T>
__host__ __device__ __forceinline__ int64_t packed_offset(int row, int k,
                                                          int K) {
  constexpr int E = Storage<T>::E, KC = Storage<T>::KC;
  const int t = row >> 4, r = row & 15, s = k / KC, g = (k % KC) / E;
  return ((((int64_t)t * (K / KC) + s) * 64 + g * 16 + r) * 16) +
         (int64_t)(k % E) * (int64_t)sizeof(T);
}

// FP8 E4M3 weights (bf16 drafters) are packed in pairs of contraction steps:
// fragment (column tile t, pair s) is 16 columns x 64 contraction elements in
// 1 KiB, lane l holding column l % 16 with bytes 0-7 = elements
// 64s + 8(l/16) .. +8 and bytes 8-15 = elements 64s + 32 + 8(l/16) .. +8, so
// one 16-byte load per lane feeds two bf16 MFMA steps (fp8x8_to_bf16 of each
// half gives the step's bf16 fragment).  Each output column's scale is
// stored in packed column order: scale[16 t + c] for column c of tile t.
__host__ __device__ __forceinline__ int64_t packed_offset_fp8(int row, int k,
                                                              int K) {
  const int t = row >> 4, r = row & 15, s = k / 64, h = (k % 64) / 32,
            g = (k % 32) / 8;
  return (((int64_t)t * (K / 64) + s) * 64 + g * 16 + r) * 16 + h * 8 + k % 8;
}

// Column order inside packed weight tiles.
enum ColMap : int {
  MAP_LINEAR = 0,  // tile t = output columns [16t, 16t + 16)
  MAP_PAIRS = 1,   // tile t = 8 "low" columns (lanes 0-7) and their partners
                   // at +pair_off (lanes 8-15); low column i is
                   // (i / pair_off) * pair_group + i % pair_off
};

__host__ __device__ __forceinline__ int map_col(int cmap, int pair_group,
                                                int pair_off, int tile,
                                                int lane16) {
  if (cmap == MAP_LINEAR) return tile * 16 + lane16;
  const int i = tile * 8 + (lane16 & 7);
  const int low = (i / pair_off) * pair_group + i % pair_off;
  return lane16 < 8 ? low : low + pair_off;
}

// What a workgroup does with its finished 16-column output tile.
enum Epilogue : int {
  EP_STORE = 0,   // out_f32 = sum (row-major)
  EP_RESID = 1,   // out_f32 += sum (the residual stream)
  EP_QKV = 2,     // q -> RoPE -> q buffer; block k -> RoPE, v -> layer cache
  EP_KV = 3,      // injected rows: k -> RoPE, v -> cache of every layer
  EP_SWIGLU = 4,  // out_t (packed, contraction I) = silu(gate) * up
  EP_TOP2 = 5,    // LM head: per row (max, argmax, 2nd max, sum exp)
};

// KV cache addressing.  Contiguous (log2 < 0): a layer's K (or V) plane is
// [max_batch][Hkv][P][d].  Paged: it is [npages][Hkv][1 << log2][d] and
// position pos of sequence seq lives in page table[seq * ld + (pos >> log2)].
struct KvPages {
  const int32_t* table = nullptr;
  int ld = 0;
  int log2 = -1;
  int npages = 0;
};
// Row (in units of d elements) of (seq, kv head h, pos) within one plane; a
// page id out of range sets DFLASH_DEVERR_PAGE and addresses page 0.
__device__ __forceinline__ int64_t kv_row(const KvPages& g, int P, int Hkv,
                                          int seq, int h, int pos, int* err) {
  if (g.log2 < 0) return ((int64_t)seq * Hkv + h) * P + pos;
  int page = g.table[(int64_t)seq * g.ld + (pos >> g.log2)];
  if (page < 0 || page >= g.npages) {
    set_error(err, DFLASH_DEVERR_PAGE);
    page = 0;
  }
  return (((int64_t)page * Hkv + h) << g.log2) + (pos & ((1 << g.log2) - 1));
}
// kv_row for a (seq, pos) that is the same across the workgroup: the page
// id is read through the constant address space, which makes it a scalar
// load, counted apart from the vector loads a pipelined loop keeps in flight
// (a vector load here would make its use wait for all of them).  The page
// table is not written while a drafting call runs.
__device__ __forceinline__ int64_t kv_row_uniform(const KvPages& g, int P,
                                                  int Hkv, int seq, int h,
                                                  int pos, int* err) {
  if (g.log2 < 0) return ((int64_t)seq * Hkv + h) * P + pos;
  typedef const int32_t __attribute__((address_space(4))) cint32;
  // the entry's address, moved to scalar registers (it is the same in
  // every lane)
  const uint64_t a =
      (uint64_t)(uintptr_t)(g.table + (int64_t)seq * g.ld + (pos >> g.log2));
  const uint64_t au =
      ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  int page = *(const cint32*)(uintptr_t)au;
  if (page < 0 || page >= g.npages) {
    set_error(err, DFLASH_DEVERR_PAGE);
    page = 0;
  }
  return (((int64_t)page * Hkv + h) << g.log2) + (pos & ((1 << g.log2) - 1));
}
// Rows of one plane.
__host__ __device__ __forceinline__ int64_t kv_plane_rows(const KvPages& g,
                                                          int max_batch,
                                                          int Hkv, int P) {
  return g.log2 < 0 ? (int64_t)max_batch * Hkv * P
                    : ((int64_t)g.npages * Hkv) << g.log2;
}

// C[M, N] = A[M, Kd] . W[N, Kd]^T.  W is packed; A is packed (a_packed) or
// row-major with up to kMaxASeg segments along the contraction (the
// concatenated target layers).  A workgroup owns one 16-column tile and 16*MT
// rows over the whole contraction, which its waves split.
struct GemmArgs {
  const void* a_ptr[kMaxASeg];
  int64_t lda;      // row-major A: row stride, elements
  int a_seg_k;      // row-major A: contraction width of each segment
  int a_packed;
  const void* w;    // packed weights [N rows][Kd]
  int wfp8;         // w holds FP8 E4M3 step pairs (packed_offset_fp8)
  const float* wscale;  // per output column, packed column order, or null
  const void* w_tiled;  // host side: the bf16 layout of FP8 weights (codes
                        // widened) for the tiled kernels, or null
  int M, N, Kd;
  int cmap, pair_group, pair_off;
  // epilogue
  int ep;
  float* out_f32;   // EP_STORE / EP_RESID rows, ld = ldo
  int64_t ldo;
  void* out_t;      // EP_QKV: q [M][Hq*d]; EP_SWIGLU: packed act
  void* kv;         // EP_QKV: this layer's cache; EP_KV: the whole cache
  const double2* rope;     // cos, sin [P][d/2]
  const int32_t* ctx_len;  // EP_QKV
  int max_len, K;
  const int32_t* row_seq;  // EP_KV
  const int32_t* row_pos;
  int Hq, Hkv, d, max_batch, P, max_ctx;
  KvPages pages;           // EP_QKV / EP_KV cache addressing
  Top2* top2;              // EP_TOP2: [M][N / 16]
  float* logits;           // EP_TOP2 debug rows (via rowmap), may be null
  const int32_t* rowmap;   //   LM-head row -> block row b*K + i, or -1
  int64_t logits_ld;
  int* err;
  // host side: the row RMSNorm that reads out_f32 next (gain, epsilon,
  // packed output), run with the split-K reduction when the GEMM is split
  // and the norm takes its row form; run_gemm sets norm_fused when it did
  const void* norm_g;
  float norm_eps;
  void* norm_out;
  int norm_fused;
};

struct GemmPlan {
  int MT, waves, gx, gy;
};
GemmPlan plan_gemm(int M, int N, bool lm_head);
hipError_t launch_gemm(bool bf16, const GemmPlan& pl, const GemmArgs& a,
                       hipStream_t s);

// LM head (EP_TOP2) of at most 16 rows as a persistent stream: returns the
// number of workgroups (> 0) when the shape is supported, else 0; the launch
// writes one top-2 record per row and workgroup, a.top2[row][parts].
int lm_head_parts(bool bf16, int M, int N, int Kd, int num_cu);
hipError_t launch_lm_head(bool bf16, int parts, const GemmArgs& a,
                          hipStream_t s);
// The FP8 gate/up projection (EP_SWIGLU, MAP_PAIRS, packed activations) of
// at most 16 rows on the same persistent stream, each tile's pairs finished
// by SwiGLU: returns the number of workgroups (> 0) when the call is
// supported and has enough tiles to keep every workgroup streaming, else 0.
int proj_stream_parts(bool bf16, const GemmArgs& a, int num_cu);
hipError_t launch_proj_stream(bool bf16, int parts, const GemmArgs& a,
                              hipStream_t s);

// Tiled MFMA GEMM for batched rows (gemm_tiled.hip): output block shapes
// rows x columns; each instance keeps its fragments in LDS per step.
enum TileCfg : int {
  TILE_64x64 = 0,
  TILE_128x128 = 1,
  TILE_256x64 = 2,
  TILE_256x128 = 3,
  TILE_128x256 = 4,
  TILE_256x256 = 5,
  TILE_256x128_W8 = 6,  // 256 x 128 on eight waves of 64 x 64
  TILE_128x192 = 7,     // 128 x 192 on four waves of 64 x 96
  TILE_128x128_W8 = 8,  // 128 x 128 on eight waves of 64 x 32
  TILE_NCFG = 9,
};
// Block shape of an M x N tiled GEMM over a contraction of Kd with epilogue
// `ep`; `splittable`: its contraction may be split (plain-store and
// residual epilogues).
int plan_tiled(int M, int N, int Kd, int ep, bool splittable);
// Top-2 records per row that the tiled LM head writes with block shape cfg
// (one per column block: top2[row * records + block]).
int tiled_top2_records(int cfg, int N);
// Output blocks of shape cfg over an M x N result.
int tiled_blocks(int cfg, int M, int N);
// bf16 only; a.a_packed must be set; a.M any size, a.N % 16 == 0,
// a.Kd % 32 == 0.  ksplit > 1 splits the contraction (EP_STORE only): copy s
// of the result goes to a.out_f32 + s * M * ldo.
hipError_t launch_gemm_tiled(bool bf16, int cfg, const GemmArgs& a,
                             int ksplit, hipStream_t s);
// out[M][N] (row stride ldo) = (out +) sum of the S planes ws[S][M][N].
hipError_t launch_splitk_reduce(int M, int N, int S, const float* ws,
                                float* out, int ldo, bool resid,
                                hipStream_t s);
// The pair epilogue (a.ep EP_QKV or EP_KV, MAP_PAIRS) of a GEMM whose S (2 to
// 4) copies were stored in tile order as ws[S][a.M][a.N] (the tiled kernel
// run with EP_STORE and MAP_LINEAR).
hipError_t launch_splitk_pair(const GemmArgs& a, int S, const float* ws,
                              hipStream_t s);
// dst = packed copy of a's row-major A segments (M rows, contraction a.Kd)
hipError_t launch_pack_act(bool bf16, const GemmArgs& a, void* dst,
                           hipStream_t s);

// Packs rows of up to kMaxBSeg row-major segments [n_s][K] (concatenated
// along rows) into dst with the given column map.
// Modes: PACK_SAME copies elements of the storage type; PACK_FP8 packs
// 1-byte E4M3 codes into step pairs; PACK_FP8_BF16 widens E4M3 codes to bf16
// in the bf16 layout; PACK_SCALE writes one float per row (the source
// segments are float vectors) in packed column order.
enum PackMode : int { PACK_SAME = 0, PACK_FP8 = 1, PACK_FP8_BF16 = 2,
                      PACK_SCALE = 3 };
struct PackArgs {
  const void* src[kMaxBSeg];
  int n0[kMaxBSeg + 1];
  int nseg;
  int N, K, cmap, pair_group, pair_off;
  int mode;
  void* dst;
};
hipError_t launch_pack(bool bf16, const PackArgs& a, hipStream_t s);

// ---- row kernels (epilogue.hip) -------------------------------------------
struct BlockState {
  int32_t* tokens;     // [B][K] current block ids
  int32_t* committed;  // [B][K] 1 = fixed
  int32_t* rowmap;     // [B * n_cap] LM-head row -> block row b*K + i, or -1
  int* err;
};

// x = E[token] (fp32); pass 0 also fills the block state; every pass
// rebuilds the LM-head row map.  With g0 != null also h0 = RMSNorm(x) * g0
// packed (the first layer's input), as launch_rmsnorm would write it.
hipError_t launch_embed(bool bf16, int B, int K, int D, int V, int mask_id,
                        int pass, int n_cap, const int32_t* anchor,
                        const int32_t* block_tokens, BlockState st,
                        const void* embed, float* x, int32_t* draft,
                        const void* g0, float eps, void* h0, hipStream_t s);

// out = RMSNorm(x[rowmap ? rowmap[r] : r]) * gain, packed (contraction D);
// rows with rowmap < 0 and rows up to the next multiple of 16 are zero.
hipError_t launch_rmsnorm(bool bf16, int rows, int D, const float* x,
                          const int32_t* rowmap, const void* gain, float eps,
                          void* out, hipStream_t s);
// Whether launch_rmsnorm takes its one-workgroup-per-row form for this shape.
bool rmsnorm_row_form(bool bf16, int rows, int D);
// The split-K reduction of S float copies ws[S][M][D] into x (added to x's
// rows when resid), fused with the row-form RMSNorm of the result into out
// (packed): the same bits as launch_splitk_reduce then launch_rmsnorm (no row
// map), for the shapes where rmsnorm_row_form holds (else an error).
hipError_t launch_splitk_norm(bool bf16, int M, int D, int S, const float* ws,
                              float* x, bool resid, const void* gain,
                              float eps, void* out, hipStream_t s);

// ---- attention (attention.hip) -----------------------------------------
struct AttnArgs {
  const void* q;        // [B*K][Hq*d] row-major
  const void* kc;       // this layer's K plane (see KvPages)
  const void* vc;       // this layer's V cache
  const int32_t* ctx_len;
  int max_len;          // host bound on ctx_len (grid sized for it)
  int P, Hq, Hkv, K;
  KvPages pages;        // cache addressing (contiguous or paged)
  int* err;             // device error word (page ids)
  int chunk, nch;       // keys per workgroup, chunks per (sequence, kv head)
  int deep;             // one workgroup per CU (long chunks): deeper staging
  int by_len;           // bf16: blockIdx.z ranks the sequences, longest first
  float scale_log2;     // log2(e) / sqrt(d)
  float* part_o;        // [B][Hq][nch][K][d]
  float* part_ml;       // [B][Hq][nch][K][2]
  void* o;              // packed [B*K rows][Hq*d]
};
hipError_t launch_attention(bool bf16, int d, int B, const AttnArgs& a,
                            hipStream_t s);

// ---- head (head.hip) -----------------------------------------------------
constexpr int kMergeChunks = 16;
// part [rows][ntiles] -> part2 [rows][kMergeChunks], merged in tile order
hipError_t launch_lm_merge(int rows, int ntiles, const Top2* part, Top2* part2,
                           hipStream_t s);
// Merges each LM-head row's nrec records (part [rows][nrec]: lm_merge's
// chunks, or the persistent LM head's per-workgroup records) and commits.
hipError_t launch_commit(int B, int K, int n_cap, int commit, bool last,
                         const Top2* part, int nrec, BlockState st,
                         int32_t* draft, float* conf, float* margin,
                         hipStream_t s);
// Speculative-sampling verification (see dflash_verify_sampling).
hipError_t launch_verify_sampling(int B, int K, int V, const int32_t* draft,
                                  const float* q, const float* p,
                                  const float* u_accept, const float* u_sample,
                                  int32_t* accept, int32_t* next,
                                  hipStream_t s);
hipError_t launch_verify(int B, int K, const int32_t* draft,
                         const int32_t* target, int32_t* accept,
                         int32_t* next_anchor, hipStream_t s);

}  // namespace dflash
