// Host side of libdflash: argument validation, workspace planning, and the
// launch sequence of each C-ABI entry point.  Nothing here computes a value
// of the method except the RoPE cos/sin table built once at create time.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
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

}  // namespace

struct dflash_ctx {
  dflash_config cfg;
  bool bf16 = true;
  size_t esz = 2;
  int num_cu = 256;
  int P = 0;  // positions per cache slot (max_ctx + block_size)

  const void* embed = nullptr;
  const void* fc = nullptr;
  const void* hidden_norm = nullptr;
  const void* final_norm = nullptr;
  const void* lm_head = nullptr;
  std::vector<const void*> attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up,
      w_down;

  void* ws = nullptr;
  size_t partial_floats = 0, attn_floats = 0, lm_part_count = 0;
  float2* rope = nullptr;
  float* partial = nullptr;
  float* x = nullptr;
  void* h = nullptr;
  void* qb = nullptr;
  void* ob = nullptr;
  void* act = nullptr;
  void* hf = nullptr;
  void* hcond = nullptr;
  int32_t* tokens = nullptr;
  int32_t* committed = nullptr;
  int32_t* rowmap = nullptr;
  Top2* lm_part = nullptr;
  RowResult* rowres = nullptr;
  float* attn_o = nullptr;
  float* attn_ml = nullptr;
  int* err = nullptr;
};

namespace {

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
  if (c->block_size != 16)
    return fail(DFLASH_E_UNSUPPORTED, "block_size %d (only 16)", c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DFLASH_E_UNSUPPORTED, "head_dim %d (64 or 128)", c->head_dim);
  if (c->dtype == DFLASH_F32 && c->head_dim != 64)
    return fail(DFLASH_E_UNSUPPORTED, "f32 drafter needs head_dim 64");
  if (c->num_q_heads % c->num_kv_heads != 0 ||
      c->num_q_heads / c->num_kv_heads > 8)
    return fail(DFLASH_E_UNSUPPORTED,
                "num_q_heads %d must be a multiple (<= 8x) of num_kv_heads %d",
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
  if (c->hidden > 16384)
    return fail(DFLASH_E_UNSUPPORTED, "hidden %d > 16384", c->hidden);
  return DFLASH_OK;
}

// Largest split-K partial buffer any call can need, over all row counts.
size_t max_partial(int max_rows, int N, int Kd, bool bf16, int num_cu) {
  size_t best = 0;
  for (int m = 16; m < max_rows + 16; m += 16) {
    const int mm = m > max_rows ? max_rows : m;
    GemmPlan pl = plan_gemm(mm, N, Kd, bf16, num_cu);
    if (pl.partial_floats > best) best = pl.partial_floats;
  }
  return best;
}

// Keys per attention workgroup: about 2 workgroups per CU over the batch,
// at least one 64-key tile each.
int attn_chunk(int B, int Hkv, int max_keys, int num_cu) {
  int target = (2 * num_cu + B * Hkv - 1) / (B * Hkv);
  if (target < 1) target = 1;
  int ch = (max_keys + target - 1) / target;
  ch = (ch + 63) / 64 * 64;
  if (ch < 64) ch = 64;
  return ch;
}

dflash_status run_gemm(dflash_ctx* c, GemmArgs& a, GemmPlan& pl,
                       hipStream_t s) {
  pl = plan_gemm(a.M, a.N, a.Kd, c->bf16, c->num_cu);
  if (pl.partial_floats > c->partial_floats)
    return fail(DFLASH_E_CAPACITY, "split-K workspace too small (%zu > %zu)",
                pl.partial_floats, c->partial_floats);
  a.k_split = pl.k_split;
  a.out = c->partial;
  DF_HIP(launch_gemm(c->bf16, pl, a, s));
  return DFLASH_OK;
}

GemmArgs make_args(const void* A, int64_t lda, int M, int Kd) {
  GemmArgs a{};
  a.a_ptr[0] = A;
  a.lda = lda;
  a.a_seg_k = Kd;
  a.M = M;
  a.Kd = Kd;
  return a;
}

void add_b(GemmArgs& a, const void* w, int n) {
  if (a.b_nseg == 0) a.b_n0[0] = 0;
  a.b_ptr[a.b_nseg] = w;
  a.b_n0[a.b_nseg + 1] = a.b_n0[a.b_nseg] + n;
  a.b_nseg++;
  a.N = a.b_n0[a.b_nseg];
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

  dflash_ctx* x = new dflash_ctx();
  x->cfg = c;
  x->bf16 = c.dtype == DFLASH_BF16;
  x->esz = x->bf16 ? 2 : 4;
  x->P = c.max_ctx + c.block_size;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&x->num_cu, hipDeviceAttributeMultiprocessorCount,
                            dev) != hipSuccess) {
    delete x;
    return fail(DFLASH_E_DEVICE, "no HIP device available");
  }
  x->embed = w->embed;
  x->fc = w->fc;
  x->hidden_norm = w->hidden_norm;
  x->final_norm = w->final_norm;
  x->lm_head = w->lm_head;
  std::vector<const void*>* dst[] = {&x->attn_norm, &x->wq, &x->wk, &x->wv,
                                     &x->wo, &x->mlp_norm, &x->w_gate,
                                     &x->w_up, &x->w_down};
  for (int i = 0; i < 9; ++i) dst[i]->assign(lists[i], lists[i] + c.num_layers);

  // ---- workspace plan ----
  const int D = c.hidden, K = c.block_size, d = c.head_dim;
  const int qd = c.num_q_heads * d, kvd = c.num_kv_heads * d;
  const int R = c.max_batch * K;
  const int TI = c.max_inject_rows;
  const bool bf = x->bf16;
  size_t pf = 0;
  auto upd = [&](size_t v) { if (v > pf) pf = v; };
  upd(max_partial(TI, D, c.num_target_layers * c.target_hidden, bf, x->num_cu));
  upd(max_partial(TI, c.num_layers * 2 * kvd, D, bf, x->num_cu));
  upd(max_partial(R, qd + 2 * kvd, D, bf, x->num_cu));
  upd(max_partial(R, D, qd, bf, x->num_cu));
  upd(max_partial(R, 2 * c.intermediate, D, bf, x->num_cu));
  upd(max_partial(R, D, c.intermediate, bf, x->num_cu));
  x->partial_floats = pf;
  const int G = c.num_q_heads / c.num_kv_heads;
  x->attn_floats = (size_t)G * (2 * x->num_cu + c.max_batch * c.num_kv_heads) * K;
  const int lm_rows = c.max_batch * (K - 1);
  x->lm_part_count = (size_t)lm_rows * ((c.vocab + 63) / 64);

  struct Item { void** p; size_t bytes; };
  std::vector<Item> items = {
      {(void**)&x->rope, (size_t)x->P * (d / 2) * sizeof(float2)},
      {(void**)&x->partial, pf * sizeof(float)},
      {(void**)&x->x, (size_t)R * D * sizeof(float)},
      {&x->h, (size_t)R * D * x->esz},
      {&x->qb, (size_t)R * qd * x->esz},
      {&x->ob, (size_t)R * qd * x->esz},
      {&x->act, (size_t)R * c.intermediate * x->esz},
      {&x->hf, (size_t)R * D * x->esz},
      {&x->hcond, (size_t)TI * D * x->esz},
      {(void**)&x->tokens, (size_t)R * sizeof(int32_t)},
      {(void**)&x->committed, (size_t)R * sizeof(int32_t)},
      {(void**)&x->rowmap, (size_t)R * sizeof(int32_t)},
      {(void**)&x->lm_part, x->lm_part_count * sizeof(Top2)},
      {(void**)&x->rowres, (size_t)lm_rows * sizeof(RowResult)},
      {(void**)&x->attn_o, x->attn_floats * d * sizeof(float)},
      {(void**)&x->attn_ml, x->attn_floats * 2 * sizeof(float)},
      {(void**)&x->err, 256},
  };
  size_t total = 0;
  for (auto& it : items) total += align_up(it.bytes, 256);
  if (hipMalloc(&x->ws, total) != hipSuccess) {
    delete x;
    return fail(DFLASH_E_DEVICE, "workspace allocation of %zu bytes failed", total);
  }
  char* p = static_cast<char*>(x->ws);
  for (auto& it : items) {
    *it.p = p;
    p += align_up(it.bytes, 256);
  }
  // RoPE table: angle pos * theta^(-2i/d) evaluated in double precision.
  std::vector<float2> tab((size_t)x->P * (d / 2));
  for (int pos = 0; pos < x->P; ++pos)
    for (int i = 0; i < d / 2; ++i) {
      const double inv = std::pow((double)c.rope_theta, -2.0 * i / d);
      const double ang = (double)pos * inv;
      tab[(size_t)pos * (d / 2) + i] = make_float2((float)std::cos(ang),
                                                   (float)std::sin(ang));
    }
  if (hipMemcpy(x->rope, tab.data(), tab.size() * sizeof(float2),
                hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(x->err, 0, 256) != hipSuccess ||
      hipMemset(x->committed, 0, (size_t)R * sizeof(int32_t)) != hipSuccess) {
    hipFree(x->ws);
    delete x;
    return fail(DFLASH_E_DEVICE, "workspace initialisation failed");
  }
  *out = x;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* ctx) {
  if (!ctx) return;
  hipDeviceSynchronize();
  if (ctx->ws) hipFree(ctx->ws);
  delete ctx;
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

  // fused features: fc over the concatenated target layers, then RMSNorm
  GemmArgs a{};
  for (int k = 0; k < c.num_target_layers; ++k) a.a_ptr[k] = target_hidden[k];
  a.lda = ld;
  a.a_seg_k = c.target_hidden;
  a.M = T;
  a.Kd = c.num_target_layers * c.target_hidden;
  add_b(a, ctx->fc, D);
  GemmPlan pl;
  dflash_status st = run_gemm(ctx, a, pl, s);
  if (st != DFLASH_OK) return st;
  DF_HIP(launch_rows_rmsnorm(ctx->bf16, T, D, pl.gz, ctx->partial,
                             ctx->hidden_norm, c.rms_eps, ctx->hcond, s));

  // every layer's K and V projection in one pass over H_cond
  GemmArgs b = make_args(ctx->hcond, D, T, D);
  for (int l = 0; l < c.num_layers; ++l) {
    add_b(b, ctx->wk[l], kvd);
    add_b(b, ctx->wv[l], kvd);
  }
  st = run_gemm(ctx, b, pl, s);
  if (st != DFLASH_OK) return st;
  DF_HIP(launch_kv_inject_epilogue(ctx->bf16, T, c.num_layers,
                                   c.num_kv_heads, d, pl.gz, ctx->partial,
                                   row_seq, row_pos, ctx->rope, c.max_batch,
                                   c.max_ctx, ctx->P, kv_cache, ctx->err, s));
  return DFLASH_OK;
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

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = ctx->bf16;
  const int D = c.hidden, d = c.head_dim, Hq = c.num_q_heads,
            Hkv = c.num_kv_heads, I = c.intermediate, V = c.vocab;
  const int qd = Hq * d, kvd = Hkv * d;
  const int R = batch * K;
  const size_t layer_elems = (size_t)2 * c.max_batch * Hkv * ctx->P * d;
  BlockState bs{ctx->tokens, ctx->committed, ctx->rowmap, ctx->err};

  AttnArgs at{};
  at.q = ctx->qb;
  at.ctx_len = ctx_len;
  at.max_len = max_ctx_len;
  at.P = ctx->P;
  at.Hq = Hq;
  at.Hkv = Hkv;
  at.K = K;
  at.chunk = attn_chunk(batch, Hkv, max_ctx_len + K, ctx->num_cu);
  at.nch = (max_ctx_len + K + at.chunk - 1) / at.chunk;
  at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  at.part_o = ctx->attn_o;
  at.part_ml = ctx->attn_ml;
  at.o = ctx->ob;
  const size_t need = (size_t)batch * Hq * at.nch * K;
  if (need > ctx->attn_floats)
    return fail(DFLASH_E_CAPACITY, "attention workspace too small");

  for (int pass = 0; pass < num_passes; ++pass) {
    const int n_cap = (K - 1) - pass * commit_per_pass;
    const bool last = pass == num_passes - 1;
    DF_HIP(launch_embed(bf, batch, K, D, V, c.mask_token_id, pass, n_cap,
                        anchor, block_tokens, bs, ctx->embed, ctx->attn_norm[0],
                        c.rms_eps, ctx->x, ctx->h, ctx->hf, draft_tokens, s));
    for (int l = 0; l < c.num_layers; ++l) {
      char* kvl = static_cast<char*>(kv_cache) + l * layer_elems * ctx->esz;
      GemmPlan pl;
      // q, k, v projection + RoPE; block k, v go to cache positions L_b + i
      GemmArgs a = make_args(ctx->h, D, R, D);
      add_b(a, ctx->wq[l], qd);
      add_b(a, ctx->wk[l], kvd);
      add_b(a, ctx->wv[l], kvd);
      dflash_status st = run_gemm(ctx, a, pl, s);
      if (st != DFLASH_OK) return st;
      DF_HIP(launch_qkv_epilogue(bf, batch, K, Hq, Hkv, d, pl.gz, ctx->partial,
                                 ctx_len, max_ctx_len, ctx->rope, ctx->P,
                                 c.max_batch, ctx->qb, kvl, ctx->err, s));
      at.kc = kvl;
      at.vc = kvl + (size_t)c.max_batch * Hkv * ctx->P * d * ctx->esz;
      DF_HIP(launch_attention(bf, d, batch, at, s));
      // output projection, residual, norm for the MLP
      GemmArgs o = make_args(ctx->ob, qd, R, qd);
      add_b(o, ctx->wo[l], D);
      st = run_gemm(ctx, o, pl, s);
      if (st != DFLASH_OK) return st;
      DF_HIP(launch_resid_norm(bf, R, K, D, pl.gz, ctx->partial, ctx->x,
                               ctx->mlp_norm[l], c.rms_eps, ctx->h, false, 0,
                               bs, s));
      // SwiGLU MLP
      GemmArgs gu = make_args(ctx->h, D, R, D);
      add_b(gu, ctx->w_gate[l], I);
      add_b(gu, ctx->w_up[l], I);
      st = run_gemm(ctx, gu, pl, s);
      if (st != DFLASH_OK) return st;
      DF_HIP(launch_swiglu(bf, R, I, pl.gz, ctx->partial, ctx->act, s));
      GemmArgs dn = make_args(ctx->act, I, R, I);
      add_b(dn, ctx->w_down[l], D);
      st = run_gemm(ctx, dn, pl, s);
      if (st != DFLASH_OK) return st;
      const bool fin = l == c.num_layers - 1;
      DF_HIP(launch_resid_norm(bf, R, K, D, pl.gz, ctx->partial, ctx->x,
                               fin ? ctx->final_norm : ctx->attn_norm[l + 1],
                               c.rms_eps, fin ? ctx->hf : ctx->h, fin, n_cap,
                               bs, s));
    }
    // LM head over the still-masked rows, fused argmax / top-2 / LSE
    const int Mh = batch * n_cap;
    GemmArgs hd = make_args(ctx->hf, D, Mh, D);
    add_b(hd, ctx->lm_head, V);
    GemmPlan hp = plan_lmhead(Mh, V, D, bf);
    float* dbg = logits_debug
                     ? logits_debug + (size_t)pass * batch * (K - 1) * V
                     : nullptr;
    DF_HIP(launch_lmhead(bf, hp, hd, ctx->lm_part, dbg, ctx->rowmap, V, s));
    DF_HIP(launch_lm_merge(Mh, hp.gx, ctx->lm_part, ctx->rowres, s));
    DF_HIP(launch_commit(batch, K, n_cap, commit_per_pass, last, ctx->rowres,
                         bs, draft_tokens, confidence, top2_margin, s));
  }
  return DFLASH_OK;
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

}  // extern "C"
