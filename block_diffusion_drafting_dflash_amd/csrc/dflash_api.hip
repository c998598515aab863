// Host side of libdflash: argument validation, workspace planning, the
// one-time weight repack, and the launch sequence of each C-ABI entry point.
// Nothing here computes a value of the method except the RoPE cos/sin table
// built once at create time.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dflash;

namespace {

thread_local std::string g_last_error;

dflash_status fail(dflash_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

#define DF_HIP(expr)                                                        \
  do {                                                                      \
    hipError_t e_ = (expr);                                                 \
    if (e_ != hipSuccess)                                                   \
      return fail(DFLASH_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr size_t kTimingSlots = 8192;
constexpr int kCommitMaxRecords = 1536;
// Timing events are bound to kernel dispatches and need no system-scope
// fence.
constexpr unsigned kTimingEventFlags = hipEventDisableSystemFence;

}  // namespace

namespace dflash {
DispatchTiming& dispatch_timing() {
  static thread_local DispatchTiming t;
  return t;
}
}  // namespace dflash

// One projection matrix in the context's layout.
struct PW {
  void* w = nullptr;        // packed: dtype fragments, or FP8 step pairs
  void* w16 = nullptr;      // FP8: codes widened to the bf16 layout, for the
                            // tiled kernels (null if no call can tile)
  float* scale = nullptr;   // FP8: per output column, packed column order
};

struct dflash_ctx {
  dflash_config cfg;
  bool bf16 = true;
  size_t esz = 2;
  int num_cu = 256;
  int device = 0;
  void* static_scratch = nullptr;  // this device's static scratch (noalloc)
  int P = 0;  // positions per cache slot (max_ctx + block_size)

  // read in place after create: the embedding table and the norm gains
  const void* embed = nullptr;
  const void* hidden_norm = nullptr;
  const void* final_norm = nullptr;
  std::vector<const void*> attn_norm, mlp_norm;

  // packed copies of every projection matrix (fragment-major, see kernels.h)
  bool fp8 = false;        // projections stored as FP8 E4M3 step pairs
  void* wpack = nullptr;
  PW pk_fc;                // [D][n_t * D_t]
  PW pk_kv;                // [N_l * 2 * Hkv * d][D], K/V heads, RoPE pairs
  PW pk_lm;                // [V][D]
  std::vector<PW> pk_qkv, pk_o, pk_gu, pk_down;

  // workspace
  void* ws = nullptr;
  size_t attn_floats = 0, lm_part_count = 0;
  double2* rope = nullptr;   // cos, sin of pos * theta^(-2i/d) [P][d/2]
  float* u = nullptr;        // fused target features before RMSNorm [TI][D]
  float* splitk = nullptr;   // split-K copies [S][rows][D]
  size_t splitk_floats = 0;
  void* cond = nullptr;      // H_cond, packed [TI16][D]
  void* hpk = nullptr;       // target hidden states, packed [TI16][n_t * D_t]
  float* x = nullptr;        // residual rows [R][D]
  void* h = nullptr;         // RMSNorm(x) * g, packed [R][D]
  void* hf = nullptr;        // final-norm rows of still-masked positions, packed
  void* qb = nullptr;        // q after RoPE [R][Hq*d]
  void* ob = nullptr;        // attention output, packed [R][Hq*d]
  void* act = nullptr;       // SwiGLU output, packed [R][I]
  int32_t* tokens = nullptr;
  int32_t* committed = nullptr;
  int32_t* rowmap = nullptr;
  Top2* lm_part = nullptr;   // [rows][V/16]
  Top2* lm_part2 = nullptr;  // [rows][kMergeChunks]
  float* attn_o = nullptr;
  float* attn_ml = nullptr;
  int* err = nullptr;

  KvPages pages;  // KV cache addressing (dflash_set_kv_pages)

  // benchmark timing of one kernel class (dflash_set_kernel_timing)
  int time_kind = 0;
  std::vector<hipEvent_t> ev_start, ev_stop;
  size_t ev_next = 0, ev_count = 0;
};

namespace {

void free_events(dflash_ctx* c) {
  for (auto e : c->ev_start) hipEventDestroy(e);
  for (auto e : c->ev_stop) hipEventDestroy(e);
  c->ev_start.clear();
  c->ev_stop.clear();
  c->ev_next = c->ev_count = 0;
}

// Arms one event pair for the `kernels` launches of the timed kernel class
// made in its scope: the first dispatch takes the start event, the last the
// stop event (launch_k), so no event sits between them.
struct TimedLaunch {
  dflash_ctx* c;
  bool on = false;
  TimedLaunch(dflash_ctx* ctx, int kind, hipStream_t, int kernels = 1)
      : c(ctx) {
    if (c->time_kind == kind && !c->ev_start.empty()) {
      on = true;
      dispatch_timing() = {c->ev_start[c->ev_next], c->ev_stop[c->ev_next],
                           kernels};
    }
  }
  ~TimedLaunch() {
    if (!on) return;
    dispatch_timing() = {};
    c->ev_next = (c->ev_next + 1) % c->ev_start.size();
    if (c->ev_count < c->ev_start.size()) c->ev_count++;
  }
};

dflash_status check_config(const dflash_config* c) {
  if (!c) return fail(DFLASH_E_INVALID, "config is NULL");
  if (c->num_layers < 1 || c->hidden < 1 || c->num_q_heads < 1 ||
      c->num_kv_heads < 1 || c->head_dim < 1 || c->intermediate < 1 ||
      c->vocab < 2 || c->num_target_layers < 1 || c->target_hidden < 1 ||
      c->block_size < 2 || c->max_batch < 1 || c->max_ctx < 1 ||
      c->max_inject_rows < 1)
    return fail(DFLASH_E_INVALID, "config has a non-positive size");
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16)
    return fail(DFLASH_E_INVALID, "unknown dtype %d", c->dtype);
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DFLASH_E_INVALID, "mask_token_id %d outside [0, %d)",
                c->mask_token_id, c->vocab);
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f))
    return fail(DFLASH_E_INVALID, "rope_theta must be > 0, rms_eps >= 0");
  if (c->weight_format != DFLASH_WEIGHTS_DTYPE &&
      c->weight_format != DFLASH_WEIGHTS_FP8_E4M3)
    return fail(DFLASH_E_INVALID, "unknown weight_format %d", c->weight_format);
  if (c->weight_format == DFLASH_WEIGHTS_FP8_E4M3 && c->dtype != DFLASH_BF16)
    return fail(DFLASH_E_UNSUPPORTED, "FP8 weights need a bf16 drafter");
  if (c->block_size != 16)
    return fail(DFLASH_E_UNSUPPORTED, "block_size %d (only 16)", c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_E_UNSUPPORTED, "head_dim %d (64 or 128)", c->head_dim);
  if (c->dtype == DFLASH_F32 && c->head_dim != 64)
    return fail(DFLASH_E_UNSUPPORTED, "f32 drafter needs head_dim 64");
  const int group = c->num_kv_heads > 0 ? c->num_q_heads / c->num_kv_heads : 0;
  if (c->num_q_heads % c->num_kv_heads != 0 ||
      (group != 2 && group != 4 && group != 8))
    return fail(DFLASH_E_UNSUPPORTED,
                "num_q_heads %d must be 2, 4 or 8 times num_kv_heads %d",
                c->num_q_heads, c->num_kv_heads);
  if (c->hidden % 64 || c->intermediate % 64 || c->target_hidden % 64 ||
      (c->num_q_heads * c->head_dim) % 64)
    return fail(DFLASH_E_UNSUPPORTED,
                "hidden, intermediate, target_hidden, Hq*d must be multiples "
                "of 64");
  if (c->vocab % 16) return fail(DFLASH_E_UNSUPPORTED, "vocab %% 16 != 0");
  if (c->num_layers > kMaxBSeg / 2)
    return fail(DFLASH_E_UNSUPPORTED, "num_layers %d > %d", c->num_layers,
                kMaxBSeg / 2);
  if (c->num_target_layers > kMaxASeg)
    return fail(DFLASH_E_UNSUPPORTED, "num_target_layers %d > %d",
                c->num_target_layers, kMaxASeg);
  const int max_hidden = c->dtype == DFLASH_F32 ? 4096 : 8192;
  if (c->hidden > max_hidden)
    return fail(DFLASH_E_UNSUPPORTED, "hidden %d > %d", c->hidden, max_hidden);
  return DFLASH_OK;
}

// Keys per attention workgroup: about DFLASH_ATTN_WG_PER_CU workgroups per
// CU over the batch, at least DFLASH_ATTN_MIN_CHUNK keys (whole 64-key tiles)
// each so that the chunk merge stays short.  Where that gives chunks of at
// least DFLASH_ATTN_LONG_CHUNK keys, one workgroup per CU with chunks twice
// as long: measured on MI355X at 32k contexts (batch 4) 106-107 against
// 112 us per launch; at 1-4k contexts two per CU stay faster (55.5 against
// 59 us).
#ifndef DFLASH_ATTN_WG_PER_CU
#define DFLASH_ATTN_WG_PER_CU 2
#endif
#ifndef DFLASH_ATTN_MIN_CHUNK
#define DFLASH_ATTN_MIN_CHUNK 128
#endif
#ifndef DFLASH_ATTN_LONG_CHUNK
#define DFLASH_ATTN_LONG_CHUNK 2048
#endif
int attn_chunk(int B, int Hkv, int max_keys, int num_cu, int* deep) {
  auto chunk_for = [&](int wg_per_cu) {
    int target = (wg_per_cu * num_cu + B * Hkv - 1) / (B * Hkv);
    if (target < 1) target = 1;
    int ch = (max_keys + target - 1) / target;
    ch = (ch + 63) / 64 * 64;
    return ch < DFLASH_ATTN_MIN_CHUNK ? DFLASH_ATTN_MIN_CHUNK : ch;
  };
  const int ch = chunk_for(DFLASH_ATTN_WG_PER_CU);
  if (ch < DFLASH_ATTN_LONG_CHUNK) {
    *deep = 0;
    return ch;
  }
  // long chunks: one workgroup per CU where the (sequence, kv head) pairs
  // leave room for it, and then the deeper staging ring of the bf16 kernel
  *deep = B * Hkv <= num_cu;
  return chunk_for(1);
}

// Up to 16 rows (and up to 64 outside the LM head) a GEMM is a weight
// stream: wide workgroups over one 16-column tile (gemm.hip).  Beyond that
// it is a dense contraction: MFMA tiles staged through LDS (gemm_tiled.hip,
// bf16 only); a row-major activation operand is packed first.
#ifndef DFLASH_PACK_ROWMAJOR
#define DFLASH_PACK_ROWMAJOR 1
#endif
// bf16 GEMMs above 64 rows are tiled; from 17 rows so are the LM head and
// wide outputs (at least DFLASH_TILED_MIN_COLS columns): there a 16-column
// streaming workgroup would re-read every activation row for each weight
// tile, while a 64-column block reads them once per 64 columns.  Narrower
// outputs keep the streaming form, which has four times the workgroups.
#ifndef DFLASH_TILED_MIN_COLS
#define DFLASH_TILED_MIN_COLS 6144
#endif
bool splittable(const GemmArgs& a) {
  return (a.ep == EP_STORE || a.ep == EP_RESID) && a.cmap == MAP_LINEAR;
}
bool gemm_is_tiled(const dflash_ctx* c, const GemmArgs& a) {
  return c->bf16 &&
         (a.M > 64 || (a.M > 16 && (a.ep == EP_TOP2 || splittable(a) ||
                                    a.N >= DFLASH_TILED_MIN_COLS)));
}

// Contraction splits of a tiled store / residual GEMM whose block grid
// leaves CUs idle: copies up to about one workgroup per CU (at most 4, at
// least 8 contraction steps each, within the split workspace).  Measured:
// at 64 rows (64 blocks, 4 copies) the split plus its reduction is 30-40%
// faster than one pass; at 256 blocks two copies gain nothing.  Copies for
// two workgroups per CU (up to 8) were slower at 64, 256 and 1024 rows
// (batch-16 step 1.72 -> 1.79 ms, batch-64 5.64 -> 5.77 ms).
#ifndef DFLASH_MAX_KSPLIT
#define DFLASH_MAX_KSPLIT 4
#endif
static_assert(DFLASH_MAX_KSPLIT >= 1 && DFLASH_MAX_KSPLIT <= 4,
              "the fused split reduction and row norm takes 1 to 4 copies");
// Where a split GEMM stores its copies: floats of room at p.
struct SplitWs {
  float* p = nullptr;
  size_t floats = 0;
};

int plan_ksplit(const dflash_ctx* c, const GemmArgs& a, int cfg,
                const SplitWs& ws) {
  if (!splittable(a)) return 1;
  const int blocks = tiled_blocks(cfg, a.M, a.N);
  int S = blocks > 0 ? c->num_cu / blocks : 1;
  S = std::min(S, DFLASH_MAX_KSPLIT);
  S = std::min(S, a.Kd / 32 / 8);
  while (S > 1 && (size_t)S * a.M * a.N > ws.floats) --S;
  return std::max(S, 1);
}

// A pair-epilogue GEMM (QKV, the injected K/V) of 65 to
// DFLASH_PAIR_SPLIT_ROWS rows whose 128 x 128 block grid fills at most half
// the CUs: that many copies over contraction ranges (at most
// DFLASH_MAX_KSPLIT, at least 8 steps each, within the split workspace),
// stored in tile order and finished by the pair reduction.  Returns the
// copies, or 1 where the GEMM keeps its unsplit plan.
#ifndef DFLASH_PAIR_SPLIT_ROWS
#define DFLASH_PAIR_SPLIT_ROWS 512
#endif
int plan_pair_split(const dflash_ctx* c, const GemmArgs& a,
                    const SplitWs& ws) {
  if ((a.ep != EP_QKV && a.ep != EP_KV) || a.cmap != MAP_PAIRS ||
      a.M <= 64 || a.M > DFLASH_PAIR_SPLIT_ROWS)
    return 1;
  const int blocks = tiled_blocks(TILE_128x128, a.M, a.N);
  int S = blocks > 0 ? c->num_cu / blocks : 1;
  S = std::min(S, DFLASH_MAX_KSPLIT);
  S = std::min(S, a.Kd / 32 / 8);
  while (S > 1 && (size_t)S * a.M * a.N > ws.floats) --S;
  return std::max(S, 1);
}

dflash_status run_gemm(dflash_ctx* c, GemmArgs& a, hipStream_t s,
                       const SplitWs& sw, int kind = DFLASH_TIME_GEMM) {
  a.err = c->err;
  const bool lm = a.ep == EP_TOP2;
  const bool tiled = gemm_is_tiled(c, a);
  if (!a.a_packed && (tiled || DFLASH_PACK_ROWMAJOR)) {
    // row-major activations (the target hidden states): pack once, so every
    // workgroup's operand loads are whole 1 KiB fragments
    DF_HIP(launch_pack_act(c->bf16, a, c->hpk, s));
    a.a_ptr[0] = c->hpk;
    a.a_packed = 1;
    a.a_seg_k = a.Kd;
  }
  if (tiled && a.wfp8) {
    // the tiled kernels take the widened codes (same values) and the scales
    if (!a.w_tiled)
      return fail(DFLASH_E_UNSUPPORTED, "no bf16 layout of the FP8 weights "
                  "for %d rows (created for fewer)", a.M);
    a.w = a.w_tiled;
    a.wfp8 = 0;
  }
  if (tiled) {
    const int ps = plan_pair_split(c, a, sw);
    if (ps > 1) {
      TimedLaunch tl(c, kind, s, 2);
      GemmArgs b = a;
      b.ep = EP_STORE;
      b.cmap = MAP_LINEAR;  // the copies in tile order
      b.out_f32 = sw.p;
      b.ldo = a.N;
      DF_HIP(launch_gemm_tiled(true, TILE_128x128, b, ps, s));
      DF_HIP(launch_splitk_pair(a, ps, sw.p, s));
      return DFLASH_OK;
    }
    const int cfg = plan_tiled(a.M, a.N, a.Kd, a.ep, splittable(a));
    const int S = plan_ksplit(c, a, cfg, sw);
    TimedLaunch tl(c, kind, s, S > 1 ? 2 : 1);
    if (S > 1) {
      // split copies into the workspace, then summed in order into the
      // output (plain store or residual add)
      GemmArgs b = a;
      b.ep = EP_STORE;
      b.out_f32 = sw.p;
      b.ldo = a.N;
      DF_HIP(launch_gemm_tiled(true, cfg, b, S, s));
      if (a.norm_g != nullptr && a.ldo == a.N &&
          rmsnorm_row_form(c->bf16, a.M, a.N)) {
        // the reduction and the row RMSNorm that reads its rows, in one pass
        DF_HIP(launch_splitk_norm(c->bf16, a.M, a.N, S, sw.p, a.out_f32,
                                  a.ep == EP_RESID, a.norm_g, a.norm_eps,
                                  a.norm_out, s));
        a.norm_fused = 1;
        return DFLASH_OK;
      }
      DF_HIP(launch_splitk_reduce(a.M, a.N, S, sw.p, a.out_f32, a.ldo,
                                  a.ep == EP_RESID, s));
      return DFLASH_OK;
    }
    DF_HIP(launch_gemm_tiled(true, cfg, a, 1, s));
    return DFLASH_OK;
  }
  if (!lm && a.a_packed) {
    const int parts = proj_stream_parts(c->bf16, a, c->num_cu);
    if (parts > 0) {
      TimedLaunch tl(c, kind, s);
      DF_HIP(launch_proj_stream(c->bf16, parts, a, s));
      return DFLASH_OK;
    }
  }
  const GemmPlan pl = plan_gemm(a.M, a.N, lm);
  TimedLaunch tl(c, kind, s);
  DF_HIP(launch_gemm(c->bf16, pl, a, s));
  return DFLASH_OK;
}

// The row RMSNorm that will read a GEMM's fp32 output: run_gemm fuses it
// with a split-K reduction where it can and then sets norm_fused.
void set_norm(GemmArgs& a, const void* gain, float eps, void* out) {
  a.norm_g = gain;
  a.norm_eps = eps;
  a.norm_out = out;
  a.norm_fused = 0;
}

// GEMM on a packed activation operand (rows M, contraction Kd).
GemmArgs packed_args(const void* A, const PW& W, bool fp8, int M, int N,
                     int Kd) {
  GemmArgs a{};
  a.a_ptr[0] = A;
  a.a_packed = 1;
  a.a_seg_k = Kd;
  a.w = W.w;
  a.wfp8 = fp8 ? 1 : 0;
  a.wscale = W.scale;
  a.w_tiled = W.w16;
  a.M = M;
  a.N = N;
  a.Kd = Kd;
  a.cmap = MAP_LINEAR;
  return a;
}

void set_pairs(GemmArgs& a, int group, int off) {
  a.cmap = MAP_PAIRS;
  a.pair_group = group;
  a.pair_off = off;
}

void set_cache_geometry(GemmArgs& a, const dflash_ctx* c) {
  a.Hq = c->cfg.num_q_heads;
  a.Hkv = c->cfg.num_kv_heads;
  a.d = c->cfg.head_dim;
  a.max_batch = c->cfg.max_batch;
  a.P = c->P;
  a.max_ctx = c->cfg.max_ctx;
  a.rope = c->rope;
  a.pages = c->pages;
}

// Per-call scratch of the drafting pass: activations, attention and LM-head
// partials, the block state between passes and the split-contraction
// copies.  The context's workspace (dflash_draft_block) or the static buffer
// (dflash_draft_block_noalloc) provides it.
struct DraftWs {
  float* x = nullptr;       // residual rows [R][D]
  void* h = nullptr;        // RMSNorm(x) * g, packed [R][D]
  void* hf = nullptr;       // final-norm rows of still-masked positions, packed
  void* qb = nullptr;       // q after RoPE [R][Hq*d]
  void* ob = nullptr;       // attention output, packed [R][Hq*d]
  void* act = nullptr;      // SwiGLU output, packed [R][I]
  int32_t* tokens = nullptr;
  int32_t* committed = nullptr;
  int32_t* rowmap = nullptr;
  Top2* lm_part = nullptr;   // [rows][V/16]
  Top2* lm_part2 = nullptr;  // [rows][kMergeChunks]
  float* attn_o = nullptr;   // [attn_rows][d]
  float* attn_ml = nullptr;  // [attn_rows][2]
  size_t attn_rows = 0;
  SplitWs split;
};

// Static scratch of the allocation-free drafting call: one copy per GPU,
// kept until the process ends.  Host code uses only the per-device address
// resolved by hipGetSymbolAddress (static_scratch_ptr), never this name.
constexpr size_t kStaticScratchBytes = DFLASH_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of `scratch` on device dev, resolved once with dev current (the
// caller has made it current); nullptr on failure.
void* static_scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Keys per attention workgroup and chunks per (sequence, kv head) for a
// call with this batch and context bound.
void attn_geometry(const dflash_ctx* c, int batch, int max_ctx_len,
                   int* chunk, int* nch, int* deep) {
  const int K = c->cfg.block_size;
  *chunk = attn_chunk(batch, c->cfg.num_kv_heads, max_ctx_len + K, c->num_cu,
                      deep);
  *nch = (max_ctx_len + K + *chunk - 1) / *chunk;
}

// Scratch of one drafting call with `batch` sequences and context bound
// max_ctx_len, carved from base (256-byte aligned pieces) when base is not
// null.  Returns the bytes used.
size_t static_layout(const dflash_ctx* c, int batch, int max_ctx_len,
                     char* base, DraftWs* ws) {
  const dflash_config& g = c->cfg;
  const int K = g.block_size, D = g.hidden, d = g.head_dim;
  const int R = batch * K, qd = g.num_q_heads * d;
  const size_t esz = c->esz;
  int chunk = 0, nch = 0;
  int deep = 0;
  attn_geometry(c, batch, max_ctx_len, &chunk, &nch, &deep);
  const size_t attn_rows = (size_t)batch * g.num_q_heads * nch * K;
  const size_t lm_rows = (size_t)batch * (K - 1);
  const size_t split_floats = (size_t)DFLASH_MAX_KSPLIT * R * D;
  struct Item { void** p; size_t bytes; };
  const Item items[] = {
      {(void**)&ws->x, (size_t)R * D * sizeof(float)},
      {&ws->h, (size_t)R * D * esz},
      {&ws->hf, (size_t)R * D * esz},
      {&ws->qb, (size_t)R * qd * esz},
      {&ws->ob, (size_t)R * qd * esz},
      {&ws->act, (size_t)R * g.intermediate * esz},
      {(void**)&ws->tokens, (size_t)R * sizeof(int32_t)},
      {(void**)&ws->committed, (size_t)R * sizeof(int32_t)},
      {(void**)&ws->rowmap, (size_t)R * sizeof(int32_t)},
      {(void**)&ws->lm_part, lm_rows * (g.vocab / 16) * sizeof(Top2)},
      {(void**)&ws->lm_part2, lm_rows * kMergeChunks * sizeof(Top2)},
      {(void**)&ws->attn_o, attn_rows * d * sizeof(float)},
      {(void**)&ws->attn_ml, attn_rows * 2 * sizeof(float)},
      {(void**)&ws->split.p, split_floats * sizeof(float)},
  };
  size_t off = 0;
  for (const Item& it : items) {
    if (base) *it.p = base + off;
    off += align_up(it.bytes, 256);
  }
  ws->attn_rows = attn_rows;
  ws->split.floats = split_floats;
  return off;
}

dflash_status check_draft_args(const dflash_ctx* ctx, int32_t batch,
                               const int32_t* anchor,
                               const int32_t* block_tokens,
                               const int32_t* ctx_len, int32_t max_ctx_len,
                               const void* kv_cache, int32_t num_passes,
                               int32_t commit_per_pass,
                               const int32_t* draft_tokens) {
  const dflash_config& c = ctx->cfg;
  const int K = c.block_size;
  if (batch < 1) return fail(DFLASH_E_SHAPE, "batch %d < 1", batch);
  if (batch > c.max_batch)
    return fail(DFLASH_E_CAPACITY, "batch %d > max_batch %d", batch,
                c.max_batch);
  if (!anchor && !block_tokens)
    return fail(DFLASH_E_INVALID, "need anchor or block_tokens");
  if (!ctx_len || !kv_cache || !draft_tokens)
    return fail(DFLASH_E_INVALID, "NULL argument");
  if (max_ctx_len < 0 || max_ctx_len > c.max_ctx)
    return fail(DFLASH_E_CAPACITY, "max_ctx_len %d outside [0, %d]",
                max_ctx_len, c.max_ctx);
  if (num_passes < 1) return fail(DFLASH_E_INVALID, "num_passes %d < 1", num_passes);
  if (num_passes > 1 &&
      (commit_per_pass < 1 || commit_per_pass * (num_passes - 1) >= K - 1))
    return fail(DFLASH_E_INVALID,
                "commit_per_pass %d invalid for %d passes (need 1 <= c and "
                "c*(S-1) < K-1)",
                commit_per_pass, num_passes);
  if (!aligned16(kv_cache))
    return fail(DFLASH_E_INVALID, "kv_cache not 16-byte aligned");
  return DFLASH_OK;
}

// The launch sequence of one drafting call on the scratch ws.
dflash_status draft_impl(dflash_ctx* ctx, const DraftWs& ws, void* stream,
                         int32_t batch, const int32_t* anchor,
                         const int32_t* block_tokens, const int32_t* ctx_len,
                         int32_t max_ctx_len, void* kv_cache,
                         int32_t num_passes, int32_t commit_per_pass,
                         int32_t* draft_tokens, float* confidence,
                         float* top2_margin, float* logits_debug) {
  dflash_status st0 = check_draft_args(ctx, batch, anchor, block_tokens,
                                       ctx_len, max_ctx_len, kv_cache,
                                       num_passes, commit_per_pass,
                                       draft_tokens);
  if (st0 != DFLASH_OK) return st0;
  const dflash_config& c = ctx->cfg;
  const int K = c.block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = ctx->bf16;
  const int D = c.hidden, d = c.head_dim, Hq = c.num_q_heads,
            Hkv = c.num_kv_heads, I = c.intermediate, V = c.vocab;
  const int qd = Hq * d, kvd = Hkv * d;
  const int R = batch * K;
  const size_t plane_elems =
      (size_t)kv_plane_rows(ctx->pages, c.max_batch, Hkv, ctx->P) * d;
  const size_t layer_elems = 2 * plane_elems;
  BlockState bs{ws.tokens, ws.committed, ws.rowmap, ctx->err};

  AttnArgs at{};
  at.pages = ctx->pages;
  at.err = ctx->err;
  at.q = ws.qb;
  at.ctx_len = ctx_len;
  at.max_len = max_ctx_len;
  at.P = ctx->P;
  at.Hq = Hq;
  at.Hkv = Hkv;
  at.K = K;
  attn_geometry(ctx, batch, max_ctx_len, &at.chunk, &at.nch, &at.deep);
  // one chunk per sequence: the ragged contexts run longest first (at batch
  // 64 with 256-2048 keys 81 against 85 us per launch; with several chunks
  // per sequence, as at batch 16, the order gained nothing)
  at.by_len = at.nch == 1 && batch > 1;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  at.part_o = ws.attn_o;
  at.part_ml = ws.attn_ml;
  at.o = ws.ob;
  const size_t need = (size_t)batch * Hq * at.nch * K;
  if (need > ws.attn_rows)
    return fail(DFLASH_E_CAPACITY, "attention workspace too small");

  for (int pass = 0; pass < num_passes; ++pass) {
    const int n_cap = (K - 1) - pass * commit_per_pass;
    const bool last = pass == num_passes - 1;
    // up to 512 rows the embedding kernel also writes the first layer's
    // normalised input (one row per workgroup is the faster form there)
    const bool fuse_norm = R <= 512;
    DF_HIP(launch_embed(bf, batch, K, D, V, c.mask_token_id, pass, n_cap,
                        anchor, block_tokens, bs, ctx->embed, ws.x,
                        draft_tokens, fuse_norm ? ctx->attn_norm[0] : nullptr,
                        c.rms_eps, ws.h, s));
    const int Nl = c.num_layers;
    bool h_ready = false;  // the previous down-projection wrote ws.h
    for (int l = 0; l < Nl; ++l) {
      char* kvl = static_cast<char*>(kv_cache) + l * layer_elems * ctx->esz;
      // q, k, v of RMSNorm(x); RoPE; q -> q buffer, block k, v -> cache
      // positions L_b + i
      if ((l > 0 || !fuse_norm) && !h_ready)
        DF_HIP(launch_rmsnorm(bf, R, D, ws.x, nullptr, ctx->attn_norm[l],
                              c.rms_eps, ws.h, s));
      h_ready = false;
      GemmArgs a = packed_args(ws.h, ctx->pk_qkv[l], ctx->fp8, R, qd + 2 * kvd, D);
      set_pairs(a, d, d / 2);
      set_cache_geometry(a, ctx);
      a.ep = EP_QKV;
      a.out_t = ws.qb;
      a.kv = kvl;
      a.ctx_len = ctx_len;
      a.max_len = max_ctx_len;
      a.K = K;
      dflash_status st = run_gemm(ctx, a, s, ws.split);
      if (st != DFLASH_OK) return st;
      at.kc = kvl;
      at.vc = kvl + plane_elems * ctx->esz;
      {
        TimedLaunch tl(ctx, DFLASH_TIME_ATTENTION, s, at.nch > 1 ? 2 : 1);
        DF_HIP(launch_attention(bf, d, batch, at, s));
      }
      // x += o . Wo^T
      GemmArgs o = packed_args(ws.ob, ctx->pk_o[l], ctx->fp8, R, D, qd);
      o.ep = EP_RESID;
      o.out_f32 = ws.x;
      o.ldo = D;
      set_norm(o, ctx->mlp_norm[l], c.rms_eps, ws.h);
      st = run_gemm(ctx, o, s, ws.split);
      if (st != DFLASH_OK) return st;
      // act = silu(h Wg^T) * (h Wu^T), h = RMSNorm(x)
      if (!o.norm_fused)
        DF_HIP(launch_rmsnorm(bf, R, D, ws.x, nullptr, ctx->mlp_norm[l],
                              c.rms_eps, ws.h, s));
      GemmArgs gu = packed_args(ws.h, ctx->pk_gu[l], ctx->fp8, R, 2 * I, D);
      set_pairs(gu, 2 * I, I);
      gu.ep = EP_SWIGLU;
      gu.out_t = ws.act;
      st = run_gemm(ctx, gu, s, ws.split);
      if (st != DFLASH_OK) return st;
      // x += act . Wd^T
      GemmArgs dn = packed_args(ws.act, ctx->pk_down[l], ctx->fp8, R, D, I);
      dn.ep = EP_RESID;
      dn.out_f32 = ws.x;
      dn.ldo = D;
      // the next layer's input norm rides on this reduction when it can
      if (l + 1 < Nl) set_norm(dn, ctx->attn_norm[l + 1], c.rms_eps, ws.h);
      st = run_gemm(ctx, dn, s, ws.split);
      if (st != DFLASH_OK) return st;
      h_ready = dn.norm_fused != 0;
    }
    // final norm of the still-masked rows (compacted), then the LM head with
    // the fused argmax / top-2 / log-sum-exp per 16-column vocabulary tile
    const int Mh = batch * n_cap;
    DF_HIP(launch_rmsnorm(bf, Mh, D, ws.x, ws.rowmap, ctx->final_norm,
                          c.rms_eps, ws.hf, s));
    GemmArgs hd = packed_args(ws.hf, ctx->pk_lm, ctx->fp8, Mh, V, D);
    hd.ep = EP_TOP2;
    hd.top2 = ws.lm_part;
    hd.rowmap = ws.rowmap;
    hd.K = K;
    hd.logits = logits_debug
                    ? logits_debug + (size_t)pass * batch * (K - 1) * V
                    : nullptr;
    hd.logits_ld = V;
    hd.err = ctx->err;
    const int parts = lm_head_parts(bf, Mh, V, D, ctx->num_cu);
    // records per row: one per workgroup of the persistent head, one per
    // column block of the tiled head, one per 16-column tile of the
    // streaming form; the commit kernel merges up to kCommitMaxRecords
    // itself
    const Top2* recs = ws.lm_part;
    int nrec = 0;
    if (parts > 0) {
      TimedLaunch tl(ctx, DFLASH_TIME_LMHEAD, s);
      DF_HIP(launch_lm_head(bf, parts, hd, s));
      nrec = parts;
    } else {
      dflash_status st = run_gemm(ctx, hd, s, ws.split, DFLASH_TIME_LMHEAD);
      if (st != DFLASH_OK) return st;
      nrec = gemm_is_tiled(ctx, hd) ? tiled_top2_records(plan_tiled(Mh, V, D, EP_TOP2, false), V)
                                    : V / 16;
      if (nrec > kCommitMaxRecords) {
        // many records per row: merge them to kMergeChunks per row first,
        // with a workgroup per (row, chunk), rather than serially per wave
        DF_HIP(launch_lm_merge(Mh, nrec, ws.lm_part, ws.lm_part2, s));
        recs = ws.lm_part2;
        nrec = kMergeChunks;
      }
    }
    DF_HIP(launch_commit(batch, K, n_cap, commit_per_pass, last, recs, nrec,
                         bs, draft_tokens, confidence, top2_margin, s));
  }
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_last_error(void) { return g_last_error.c_str(); }

size_t dflash_kv_cache_bytes(const dflash_config* c) {
  if (!c || c->num_layers < 1 || c->max_batch < 1 || c->max_ctx < 1) return 0;
  const size_t esz = c->dtype == DFLASH_F32 ? 4 : 2;
  return (size_t)c->num_layers * 2 * c->max_batch * c->num_kv_heads *
         (size_t)(c->max_ctx + c->block_size) * c->head_dim * esz;
}

size_t dflash_kv_cache_paged_bytes(const dflash_config* c, int32_t page_size,
                                   int32_t num_pages) {
  if (!c || c->num_layers < 1 || page_size < 1 || num_pages < 1) return 0;
  const size_t esz = c->dtype == DFLASH_F32 ? 4 : 2;
  return (size_t)c->num_layers * 2 * num_pages * c->num_kv_heads *
         (size_t)page_size * c->head_dim * esz;
}

dflash_status dflash_set_kv_pages(dflash_ctx* ctx, int32_t page_size,
                                  int32_t num_pages,
                                  const int32_t* block_table,
                                  int32_t table_ld) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  if (page_size == 0) {
    ctx->pages = KvPages{};
    return DFLASH_OK;
  }
  int log2 = 0;
  while ((1 << log2) < page_size && log2 < 30) ++log2;
  if (page_size < 64 || (1 << log2) != page_size)
    return fail(DFLASH_E_SHAPE,
                "page_size %d: a power of two of at least 64 (or 0)", page_size);
  if (num_pages < 1) return fail(DFLASH_E_SHAPE, "num_pages %d < 1", num_pages);
  if (!block_table) return fail(DFLASH_E_INVALID, "block_table is NULL");
  const int64_t cap = (int64_t)table_ld * page_size;
  if (table_ld < 1 || cap < ctx->P)
    return fail(DFLASH_E_SHAPE,
                "table_ld %d pages of %d positions < max_ctx + block_size %d",
                table_ld, page_size, ctx->P);
  ctx->pages.table = block_table;
  ctx->pages.ld = table_ld;
  ctx->pages.log2 = log2;
  ctx->pages.npages = num_pages;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* ctx) {
  if (!ctx) return;
  hipDeviceSynchronize();
  free_events(ctx);
  if (ctx->ws) hipFree(ctx->ws);
  if (ctx->wpack) hipFree(ctx->wpack);
  delete ctx;
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w,
                            dflash_ctx** out) {
  g_last_error.clear();
  if (!out) return fail(DFLASH_E_INVALID, "out is NULL");
  *out = nullptr;
  dflash_status st = check_config(cfg);
  if (st != DFLASH_OK) return st;
  if (!w) return fail(DFLASH_E_INVALID, "weights is NULL");
  const dflash_config& c = *cfg;
  const void* singles[] = {w->embed, w->fc, w->hidden_norm, w->final_norm,
                           w->lm_head};
  const char* names[] = {"embed", "fc", "hidden_norm", "final_norm", "lm_head"};
  for (int i = 0; i < 5; ++i) {
    if (!singles[i]) return fail(DFLASH_E_INVALID, "weight %s is NULL", names[i]);
    if (!aligned16(singles[i]))
      return fail(DFLASH_E_INVALID, "weight %s not 16-byte aligned", names[i]);
  }
  const void* const* lists[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo,
                                w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  const char* lnames[] = {"attn_norm", "wq", "wk", "wv", "wo",
                          "mlp_norm", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 9; ++i) {
    if (!lists[i]) return fail(DFLASH_E_INVALID, "weight list %s is NULL", lnames[i]);
    for (int l = 0; l < c.num_layers; ++l) {
      if (!lists[i][l])
        return fail(DFLASH_E_INVALID, "weight %s[%d] is NULL", lnames[i], l);
      if (!aligned16(lists[i][l]))
        return fail(DFLASH_E_INVALID, "weight %s[%d] not 16-byte aligned",
                    lnames[i], l);
    }
  }

  if (c.weight_format == DFLASH_WEIGHTS_FP8_E4M3) {
    const float* sing[] = {w->fc_scale, w->lm_head_scale};
    const char* sn[] = {"fc_scale", "lm_head_scale"};
    for (int i = 0; i < 2; ++i)
      if (!sing[i] || (reinterpret_cast<uintptr_t>(sing[i]) & 3u))
        return fail(DFLASH_E_INVALID, "FP8 weights: %s NULL or misaligned",
                    sn[i]);
    const float* const* sl[] = {w->wq_scale, w->wk_scale, w->wv_scale,
                                w->wo_scale, w->w_gate_scale, w->w_up_scale,
                                w->w_down_scale};
    const char* sln[] = {"wq_scale", "wk_scale", "wv_scale", "wo_scale",
                         "w_gate_scale", "w_up_scale", "w_down_scale"};
    for (int i = 0; i < 7; ++i) {
      if (!sl[i]) return fail(DFLASH_E_INVALID, "FP8 weights: %s is NULL", sln[i]);
      for (int l = 0; l < c.num_layers; ++l)
        if (!sl[i][l] || (reinterpret_cast<uintptr_t>(sl[i][l]) & 3u))
          return fail(DFLASH_E_INVALID, "FP8 weights: %s[%d] NULL or "
                      "misaligned", sln[i], l);
    }
  }

  dflash_ctx* x = new dflash_ctx();
  x->cfg = c;
  x->bf16 = c.dtype == DFLASH_BF16;
  x->fp8 = c.weight_format == DFLASH_WEIGHTS_FP8_E4M3;
  x->esz = x->bf16 ? 2 : 4;
  x->P = c.max_ctx + c.block_size;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&x->num_cu, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess) {
    delete x;
    return fail(DFLASH_E_DEVICE, "no HIP device available");
  }
  x->device = dev;
  // the allocation-free drafting call's scratch on this device (resolved
  // once per device, with the device current)
  x->static_scratch = static_scratch_ptr(dev);
  if (!x->static_scratch) {
    delete x;
    return fail(DFLASH_E_DEVICE, "hipGetSymbolAddress of the static scratch "
                "failed on device %d", dev);
  }
  x->embed = w->embed;
  x->hidden_norm = w->hidden_norm;
  x->final_norm = w->final_norm;
  x->attn_norm.assign(w->attn_norm, w->attn_norm + c.num_layers);
  x->mlp_norm.assign(w->mlp_norm, w->mlp_norm + c.num_layers);

  const int D = c.hidden, K = c.block_size, d = c.head_dim, I = c.intermediate;
  const int qd = c.num_q_heads * d, kvd = c.num_kv_heads * d;
  const int ntd = c.num_target_layers * c.target_hidden;
  const int Nl = c.num_layers;
  const size_t esz = x->esz;

  // ---- packed weights: one allocation, repacked by pack kernels ----
  // One entry per projection matrix: its packed form (dtype fragments, or
  // FP8 step pairs), and with FP8 weights the per-column scales and, where
  // some call can run the tiled kernels, the codes widened to the bf16
  // layout (inject above 16 rows, drafting batches above one sequence).
  const bool fp8 = x->fp8;
  const bool w16_inject = fp8 && c.max_inject_rows > 16;
  const bool w16_draft = fp8 && c.max_batch > 1;
  struct PItem { PW* pw; size_t rows, cols; bool w16; };
  std::vector<PItem> pit;
  x->pk_qkv.resize(Nl);
  x->pk_o.resize(Nl);
  x->pk_gu.resize(Nl);
  x->pk_down.resize(Nl);
  pit.push_back({&x->pk_fc, (size_t)D, (size_t)ntd, w16_inject});
  pit.push_back({&x->pk_kv, (size_t)Nl * 2 * kvd, (size_t)D, w16_inject});
  pit.push_back({&x->pk_lm, (size_t)c.vocab, (size_t)D, w16_draft});
  for (int l = 0; l < Nl; ++l) {
    pit.push_back({&x->pk_qkv[l], (size_t)(qd + 2 * kvd), (size_t)D, w16_draft});
    pit.push_back({&x->pk_o[l], (size_t)D, (size_t)qd, w16_draft});
    pit.push_back({&x->pk_gu[l], (size_t)2 * I, (size_t)D, w16_draft});
    pit.push_back({&x->pk_down[l], (size_t)D, (size_t)I, w16_draft});
  }
  const size_t wsz = fp8 ? 1 : esz;
  size_t ptotal = 0;
  for (auto& it : pit) {
    ptotal += align_up(it.rows * it.cols * wsz, 256);
    if (fp8) ptotal += align_up(it.rows * sizeof(float), 256);
    if (it.w16) ptotal += align_up(it.rows * it.cols * 2, 256);
  }
  if (hipMalloc(&x->wpack, ptotal) != hipSuccess) {
    delete x;
    return fail(DFLASH_E_DEVICE, "packed-weight allocation of %zu bytes failed",
                ptotal);
  }
  {
    char* p = static_cast<char*>(x->wpack);
    for (auto& it : pit) {
      it.pw->w = p;
      p += align_up(it.rows * it.cols * wsz, 256);
      if (fp8) {
        it.pw->scale = reinterpret_cast<float*>(p);
        p += align_up(it.rows * sizeof(float), 256);
      }
      if (it.w16) {
        it.pw->w16 = p;
        p += align_up(it.rows * it.cols * 2, 256);
      }
    }
  }
  using Segs = std::vector<std::pair<const void*, int>>;
  auto pack1 = [&](const Segs& segs, int Kd, void* dst, int cmap, int group,
                   int off, int mode) -> bool {
    PackArgs a{};
    int n = 0;
    a.n0[0] = 0;
    for (auto& sg : segs) {
      a.src[a.nseg] = sg.first;
      n += sg.second;
      a.n0[++a.nseg] = n;
    }
    a.N = n;
    a.K = Kd;
    a.cmap = cmap;
    a.pair_group = group;
    a.pair_off = off;
    a.mode = mode;
    a.dst = dst;
    return launch_pack(x->bf16, a, nullptr) == hipSuccess;
  };
  // a matrix from its row segments (and, FP8, their scale vectors)
  auto pack = [&](const Segs& segs, const Segs& scales, int Kd, PW& pw,
                  int cmap, int group, int off) -> bool {
    if (!fp8) return pack1(segs, Kd, pw.w, cmap, group, off, PACK_SAME);
    return pack1(segs, Kd, pw.w, cmap, group, off, PACK_FP8) &&
           pack1(scales, 1, pw.scale, cmap, group, off, PACK_SCALE) &&
           (!pw.w16 ||
            pack1(segs, Kd, pw.w16, cmap, group, off, PACK_FP8_BF16));
  };
  bool ok = pack({{w->fc, D}}, {{w->fc_scale, D}}, ntd, x->pk_fc, MAP_LINEAR,
                 0, 0) &&
            pack({{w->lm_head, c.vocab}}, {{w->lm_head_scale, c.vocab}}, D,
                 x->pk_lm, MAP_LINEAR, 0, 0);
  {
    Segs kvsegs, kvsc;
    for (int l = 0; l < Nl; ++l) {
      kvsegs.push_back({w->wk[l], kvd});
      kvsegs.push_back({w->wv[l], kvd});
      if (fp8) {
        kvsc.push_back({w->wk_scale[l], kvd});
        kvsc.push_back({w->wv_scale[l], kvd});
      }
    }
    ok = ok && pack(kvsegs, kvsc, D, x->pk_kv, MAP_PAIRS, d, d / 2);
  }
  for (int l = 0; l < Nl && ok; ++l) {
    auto sc = [&](const float* const* v, int n) -> std::pair<const void*, int> {
      return {fp8 ? v[l] : nullptr, n};
    };
    ok = pack({{w->wq[l], qd}, {w->wk[l], kvd}, {w->wv[l], kvd}},
              {sc(w->wq_scale, qd), sc(w->wk_scale, kvd),
               sc(w->wv_scale, kvd)},
              D, x->pk_qkv[l], MAP_PAIRS, d, d / 2) &&
         pack({{w->wo[l], D}}, {sc(w->wo_scale, D)}, qd, x->pk_o[l],
              MAP_LINEAR, 0, 0) &&
         pack({{w->w_gate[l], I}, {w->w_up[l], I}},
              {sc(w->w_gate_scale, I), sc(w->w_up_scale, I)}, D, x->pk_gu[l],
              MAP_PAIRS, 2 * I, I) &&
         pack({{w->w_down[l], D}}, {sc(w->w_down_scale, D)}, I,
              x->pk_down[l], MAP_LINEAR, 0, 0);
  }
  if (!ok || hipDeviceSynchronize() != hipSuccess) {
    dflash_destroy(x);
    return fail(DFLASH_E_DEVICE, "weight repack failed");
  }

  // ---- workspace ----
  const int R = c.max_batch * K;
  const int TI = c.max_inject_rows;
  const int TI16 = (TI + 15) / 16 * 16;
  const int G = c.num_q_heads / c.num_kv_heads;
  x->attn_floats =
      (size_t)G * (DFLASH_ATTN_WG_PER_CU * x->num_cu + c.max_batch * c.num_kv_heads) * K;
  x->splitk_floats = (size_t)DFLASH_MAX_KSPLIT * std::max(R, TI16) * D;
  const int lm_rows = c.max_batch * (K - 1);
  x->lm_part_count = (size_t)lm_rows * (c.vocab / 16);

  struct Item { void** p; size_t bytes; };
  std::vector<Item> items = {
      {(void**)&x->rope, (size_t)x->P * (d / 2) * sizeof(double2)},
      {(void**)&x->u, (size_t)TI * D * sizeof(float)},
      {(void**)&x->splitk, x->splitk_floats * sizeof(float)},
      {&x->cond, (size_t)TI16 * D * esz},
      {&x->hpk, (size_t)TI16 * c.num_target_layers * c.target_hidden * esz},
      {(void**)&x->x, (size_t)R * D * sizeof(float)},
      {&x->h, (size_t)R * D * esz},
      {&x->hf, (size_t)R * D * esz},
      {&x->qb, (size_t)R * qd * esz},
      {&x->ob, (size_t)R * qd * esz},
      {&x->act, (size_t)R * I * esz},
      {(void**)&x->tokens, (size_t)R * sizeof(int32_t)},
      {(void**)&x->committed, (size_t)R * sizeof(int32_t)},
      {(void**)&x->rowmap, (size_t)R * sizeof(int32_t)},
      {(void**)&x->lm_part, x->lm_part_count * sizeof(Top2)},
      {(void**)&x->lm_part2, (size_t)lm_rows * kMergeChunks * sizeof(Top2)},
      {(void**)&x->attn_o, x->attn_floats * d * sizeof(float)},
      {(void**)&x->attn_ml, x->attn_floats * 2 * sizeof(float)},
      {(void**)&x->err, 256},
  };
  size_t total = 0;
  for (auto& it : items) total += align_up(it.bytes, 256);
  if (hipMalloc(&x->ws, total) != hipSuccess) {
    dflash_destroy(x);
    return fail(DFLASH_E_DEVICE, "workspace allocation of %zu bytes failed", total);
  }
  {
    char* p = static_cast<char*>(x->ws);
    for (auto& it : items) {
      *it.p = p;
      p += align_up(it.bytes, 256);
    }
  }
  // RoPE table: angle pos * theta^(-2i/d) evaluated in double precision.
  std::vector<double2> tab((size_t)x->P * (d / 2));
  for (int pos = 0; pos < x->P; ++pos)
    for (int i = 0; i < d / 2; ++i) {
      const double inv = std::pow((double)c.rope_theta, -2.0 * i / d);
      const double ang = (double)pos * inv;
      tab[(size_t)pos * (d / 2) + i] = make_double2(std::cos(ang), std::sin(ang));
    }
  if (hipMemcpy(x->rope, tab.data(), tab.size() * sizeof(double2),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(x->err, 0, 256) != hipSuccess ||
      hipMemset(x->committed, 0, (size_t)R * sizeof(int32_t)) != hipSuccess) {
    dflash_destroy(x);
    return fail(DFLASH_E_DEVICE, "workspace initialisation failed");
  }
  *out = x;
  return DFLASH_OK;
}

dflash_status dflash_set_kernel_timing(dflash_ctx* ctx, int32_t kind) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  if (kind < 0 || kind > DFLASH_TIME_GEMM)
    return fail(DFLASH_E_INVALID, "unknown timing kind %d", kind);
  DF_HIP(hipDeviceSynchronize());
  free_events(ctx);
  ctx->time_kind = kind;
  if (kind == 0) return DFLASH_OK;
  ctx->ev_start.resize(kTimingSlots);
  ctx->ev_stop.resize(kTimingSlots);
  for (size_t i = 0; i < kTimingSlots; ++i) {
    if (hipEventCreateWithFlags(&ctx->ev_start[i], kTimingEventFlags) != hipSuccess ||
        hipEventCreateWithFlags(&ctx->ev_stop[i], kTimingEventFlags) != hipSuccess) {
      ctx->ev_start.resize(i);
      ctx->ev_stop.resize(i);
      free_events(ctx);
      ctx->time_kind = 0;
      return fail(DFLASH_E_DEVICE, "hipEventCreate failed");
    }
  }
  return DFLASH_OK;
}

dflash_status dflash_get_kernel_timing(dflash_ctx* ctx, int32_t* launches,
                                       double* total_ms) {
  g_last_error.clear();
  if (!ctx || !launches || !total_ms)
    return fail(DFLASH_E_INVALID, "NULL argument");
  double tot = 0.0;
  const size_t n = ctx->ev_count, cap = ctx->ev_start.size();
  for (size_t k = 0; k < n; ++k) {
    const size_t i = (ctx->ev_next + cap - n + k) % cap;
    DF_HIP(hipEventSynchronize(ctx->ev_stop[i]));
    float ms = 0.f;
    DF_HIP(hipEventElapsedTime(&ms, ctx->ev_start[i], ctx->ev_stop[i]));
    tot += ms;
  }
  *launches = (int32_t)n;
  *total_ms = tot;
  ctx->ev_count = 0;
  return DFLASH_OK;
}

dflash_status dflash_check_device_errors(dflash_ctx* ctx, void* stream,
                                         int32_t* bits) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  DF_HIP(hipStreamSynchronize(s));
  int v = 0;
  DF_HIP(hipMemcpy(&v, ctx->err, sizeof(int), hipMemcpyDeviceToHost));
  if (bits) *bits = v;
  if (v != 0) {
    DF_HIP(hipMemset(ctx->err, 0, sizeof(int)));
    return fail(DFLASH_E_DEVICE, "device error bits 0x%x", v);
  }
  return DFLASH_OK;
}

dflash_status dflash_inject_kv(dflash_ctx* ctx, void* stream,
                               const void* const* target_hidden, int64_t ld,
                               int32_t T, const int32_t* row_seq,
                               const int32_t* row_pos, void* kv_cache) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  const dflash_config& c = ctx->cfg;
  if (!target_hidden || !row_seq || !row_pos || !kv_cache)
    return fail(DFLASH_E_INVALID, "NULL argument");
  if (T < 1) return fail(DFLASH_E_SHAPE, "T = %d < 1", T);
  if (T > c.max_inject_rows)
    return fail(DFLASH_E_CAPACITY, "T = %d > max_inject_rows %d", T,
                c.max_inject_rows);
  if (ld < c.target_hidden)
    return fail(DFLASH_E_SHAPE, "ld %lld < target_hidden %d", (long long)ld,
                c.target_hidden);
  if ((ld * (int64_t)ctx->esz) % 16)
    return fail(DFLASH_E_INVALID, "row stride must be a multiple of 16 bytes");
  for (int k = 0; k < c.num_target_layers; ++k) {
    if (!target_hidden[k])
      return fail(DFLASH_E_INVALID, "target_hidden[%d] is NULL", k);
    if (!aligned16(target_hidden[k]))
      return fail(DFLASH_E_INVALID, "target_hidden[%d] not 16-byte aligned", k);
  }
  if (!aligned16(kv_cache))
    return fail(DFLASH_E_INVALID, "kv_cache not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = c.hidden, d = c.head_dim, kvd = c.num_kv_heads * d;
  const int ntd = c.num_target_layers * c.target_hidden;

  // fused features: u = fc . concat(target layers), A read row-major from
  // the caller's hidden states
  GemmArgs a{};
  for (int k = 0; k < c.num_target_layers; ++k) a.a_ptr[k] = target_hidden[k];
  a.lda = ld;
  a.a_seg_k = c.target_hidden;
  a.a_packed = 0;
  a.w = ctx->pk_fc.w;
  a.wfp8 = ctx->fp8 ? 1 : 0;
  a.wscale = ctx->pk_fc.scale;
  a.w_tiled = ctx->pk_fc.w16;
  a.M = T;
  a.N = D;
  a.Kd = ntd;
  a.cmap = MAP_LINEAR;
  a.ep = EP_STORE;
  a.out_f32 = ctx->u;
  a.ldo = D;
  set_norm(a, ctx->hidden_norm, c.rms_eps, ctx->cond);
  const SplitWs sw{ctx->splitk, ctx->splitk_floats};
  dflash_status st = run_gemm(ctx, a, s, sw);
  if (st != DFLASH_OK) return st;
  // H_cond = RMSNorm(u) * g
  if (!a.norm_fused)
    DF_HIP(launch_rmsnorm(ctx->bf16, T, D, ctx->u, nullptr, ctx->hidden_norm,
                          c.rms_eps, ctx->cond, s));
  // every layer's K and V projection of H_cond in one pass; RoPE on K;
  // scatter into the cache
  GemmArgs b = packed_args(ctx->cond, ctx->pk_kv, ctx->fp8, T, c.num_layers * 2 * kvd, D);
  set_pairs(b, d, d / 2);
  set_cache_geometry(b, ctx);
  b.ep = EP_KV;
  b.kv = kv_cache;
  b.row_seq = row_seq;
  b.row_pos = row_pos;
  return run_gemm(ctx, b, s, sw);
}

dflash_status dflash_draft_block(dflash_ctx* ctx, void* stream, int32_t batch,
                                 const int32_t* anchor,
                                 const int32_t* block_tokens,
                                 const int32_t* ctx_len, int32_t max_ctx_len,
                                 void* kv_cache, int32_t num_passes,
                                 int32_t commit_per_pass,
                                 int32_t* draft_tokens, float* confidence,
                                 float* top2_margin, float* logits_debug) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  DraftWs ws;
  ws.x = ctx->x;
  ws.h = ctx->h;
  ws.hf = ctx->hf;
  ws.qb = ctx->qb;
  ws.ob = ctx->ob;
  ws.act = ctx->act;
  ws.tokens = ctx->tokens;
  ws.committed = ctx->committed;
  ws.rowmap = ctx->rowmap;
  ws.lm_part = ctx->lm_part;
  ws.lm_part2 = ctx->lm_part2;
  ws.attn_o = ctx->attn_o;
  ws.attn_ml = ctx->attn_ml;
  ws.attn_rows = ctx->attn_floats;
  ws.split = SplitWs{ctx->splitk, ctx->splitk_floats};
  return draft_impl(ctx, ws, stream, batch, anchor, block_tokens, ctx_len,
                    max_ctx_len, kv_cache, num_passes, commit_per_pass,
                    draft_tokens, confidence, top2_margin, logits_debug);
}

dflash_status dflash_draft_block_noalloc(
    dflash_ctx* ctx, void* stream, int32_t batch, const int32_t* anchor,
    const int32_t* block_tokens, const int32_t* ctx_len, int32_t max_ctx_len,
    void* kv_cache, int32_t num_passes, int32_t commit_per_pass,
    int32_t* draft_tokens, float* confidence, float* top2_margin,
    float* logits_debug) {
  g_last_error.clear();
  if (!ctx) return fail(DFLASH_E_INVALID, "ctx is NULL");
  dflash_status st = check_draft_args(ctx, batch, anchor, block_tokens,
                                      ctx_len, max_ctx_len, kv_cache,
                                      num_passes, commit_per_pass,
                                      draft_tokens);
  if (st != DFLASH_OK) return st;
  char* base = static_cast<char*>(ctx->static_scratch);
  if (!base)
    return fail(DFLASH_E_DEVICE, "static scratch of device %d not resolved",
                ctx->device);
  DraftWs ws;
  const size_t need = static_layout(ctx, batch, max_ctx_len, nullptr, &ws);
  if (need > kStaticScratchBytes)
    return fail(DFLASH_E_CAPACITY,
                "batch %d with max_ctx_len %d needs %zu bytes of scratch, "
                "more than the %zu of the static buffer",
                batch, max_ctx_len, need, (size_t)kStaticScratchBytes);
  static_layout(ctx, batch, max_ctx_len, base, &ws);
  return draft_impl(ctx, ws, stream, batch, anchor, block_tokens, ctx_len,
                    max_ctx_len, kv_cache, num_passes, commit_per_pass,
                    draft_tokens, confidence, top2_margin, logits_debug);
}

dflash_status dflash_verify_greedy(void* stream, int32_t batch,
                                   int32_t block_size,
                                   const int32_t* draft_tokens,
                                   const int32_t* target_argmax,
                                   int32_t* accept_len, int32_t* next_anchor) {
  g_last_error.clear();
  if (batch < 1) return fail(DFLASH_E_SHAPE, "batch %d < 1", batch);
  if (block_size < 1 || block_size > 64)
    return fail(DFLASH_E_SHAPE, "block_size %d outside [1, 64]", block_size);
  if (!draft_tokens || !target_argmax || !accept_len || !next_anchor)
    return fail(DFLASH_E_INVALID, "NULL argument");
  DF_HIP(launch_verify(batch, block_size, draft_tokens, target_argmax,
                       accept_len, next_anchor,
                       static_cast<hipStream_t>(stream)));
  return DFLASH_OK;
}

dflash_status dflash_verify_sampling(void* stream, int32_t batch,
                                     int32_t block_size, int32_t vocab,
                                     const int32_t* draft_tokens,
                                     const float* draft_probs,
                                     const float* target_probs,
                                     const float* u_accept,
                                     const float* u_sample,
                                     int32_t* accept_len,
                                     int32_t* next_token) {
  g_last_error.clear();
  if (batch < 1) return fail(DFLASH_E_SHAPE, "batch %d < 1", batch);
  if (block_size < 2 || block_size > 64)
    return fail(DFLASH_E_SHAPE, "block_size %d outside [2, 64]", block_size);
  if (vocab < 1 || vocab > 262144)
    return fail(DFLASH_E_SHAPE, "vocab %d outside [1, 262144]", vocab);
  if (!draft_tokens || !draft_probs || !target_probs || !u_accept ||
      !u_sample || !accept_len || !next_token)
    return fail(DFLASH_E_INVALID, "NULL argument");
  DF_HIP(launch_verify_sampling(batch, block_size, vocab, draft_tokens,
                                draft_probs, target_probs, u_accept, u_sample,
                                accept_len, next_token,
                                static_cast<hipStream_t>(stream)));
  return DFLASH_OK;
}

}  // extern "C"
