/*
 * dflash.h -- C ABI of the DFlash drafting hot path on AMD Instinct MI355X
 * (gfx950).
 *
 * One drafting step of DFlash block-diffusion speculative decoding:
 *   dflash_inject_kv     target hidden states from several target layers are
 *                        fused (concat -> fc -> RMSNorm) and projected through
 *                        every draft layer's K/V weights (RoPE on K) into the
 *                        draft KV cache;
 *   dflash_draft_block   a block of K = 16 positions (the anchor, then K-1
 *                        mask tokens) runs once through every draft layer and
 *                        the LM head; each masked position takes its argmax
 *                        (optionally over S confidence-ordered refinement
 *                        passes);
 *   dflash_verify_greedy the accepted length is the longest prefix of the
 *                        draft that matches the target's greedy tokens, plus
 *                        one token from the target;
 *   dflash_verify_sampling
 *                        the same for sampled decoding (temperature > 0):
 *                        lossless speculative-sampling acceptance against the
 *                        draft's and the target's probabilities.
 *
 * Sources: "DFlash Guide: Block Diffusion for Speculative Decoding"
 * (aifetchly blog), "DFlash: Block Diffusion for Flash Speculative Decoding"
 * (sciencestack abstract page, arXiv 2602.06036) and "DFlash: Diffusion Drafts
 * the Block" (stable-lab tutorial).  Each entry point cites its passage.
 *
 * Conventions for every call:
 *   - All tensor arguments are DEVICE pointers unless marked "host".  The
 *     caller owns every weight, input, output and the KV cache; the library
 *     never frees them.  Weights are read-only.  Tensor pointers must be
 *     16-byte aligned.
 *   - Element type of weights, hidden states, activations and the KV cache is
 *     the config's dtype (DFLASH_BF16 or DFLASH_F32); ids are int32; logits,
 *     confidences and margins are fp32.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  They allocate nothing, synchronise nothing and read nothing
 *     back to the host, so a step can be enqueued without host stalls.
 *     Lengths live in device arrays; the host passes only upper bounds that
 *     size the launch grids.
 *   - Host-side validation runs before anything is launched.  A failing call
 *     launches nothing and returns a negative dflash_status;
 *     dflash_last_error() then returns a message (per thread).
 *   - Values that only the device sees (an out-of-range token id, context
 *     length, slot or position) are clamped so that every access stays in
 *     bounds, and set a sticky device error word that
 *     dflash_check_device_errors() reports.
 *   - Results are bitwise reproducible from run to run: no reduction depends
 *     on scheduling order.
 *   - A context's workspace (activations, partial sums, split-contraction
 *     copies, the block state between passes) is shared by all its calls, so
 *     calls on one context must not overlap: issue them on one stream, or
 *     order the streams.  Different contexts are independent.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,     /* null pointer, misaligned pointer, bad scalar */
  DFLASH_E_SHAPE = -2,       /* sizes inconsistent with each other */
  DFLASH_E_CAPACITY = -3,    /* beyond max_batch / max_ctx / max_inject_rows */
  DFLASH_E_DEVICE = -4,      /* HIP runtime failure or device error word set */
  DFLASH_E_UNSUPPORTED = -5  /* a shape the kernels do not implement */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Storage of the projection matrices (fc, wq, wk, wv, wo, w_gate, w_up,
 * w_down, lm_head).  DFLASH_WEIGHTS_DTYPE: the config dtype.
 * DFLASH_WEIGHTS_FP8_E4M3 (bf16 drafters): one byte per element, the OCP
 * FP8 E4M3 code (1 sign, 4 exponent bits of bias 7, 3 mantissa bits; codes
 * 0x7F/0xFF are NaN and must not occur), with one fp32 scale per output
 * row: W[j][k] = scale[j] * value(code[j][k]).  Activations stay bf16 and
 * every row's sum is scaled once, in fp32 or wider, before it is stored.
 * The embedding and the norm gains stay in the config dtype.  This is the
 * FP8 drafter-weight execution of "DFlash Guide", section "Production
 * Benchmarks on NVIDIA Blackwell B200" (FP4/FP8 mixed execution; the page
 * fixes no format, this is the reading taken). */
typedef enum {
  DFLASH_WEIGHTS_DTYPE = 0,
  DFLASH_WEIGHTS_FP8_E4M3 = 1
} dflash_weight_format;

/* Device error word bits (dflash_check_device_errors). */
#define DFLASH_DEVERR_TOKEN    0x1  /* token id outside [0, vocab), or a drafted position whose logits had no finite maximum (id -1) */
#define DFLASH_DEVERR_CTX_LEN  0x2  /* context length outside [0, max_ctx_len] */
#define DFLASH_DEVERR_SLOT     0x4  /* inject row's sequence slot out of range */
#define DFLASH_DEVERR_POS      0x8  /* inject row's position out of range */
#define DFLASH_DEVERR_PAGE     0x10 /* KV page id outside [0, num_pages) */

/* Drafter shape and capacities.  Supported: block_size == 16; head_dim 64 or
 * 128; num_q_heads equal to 2, 4 or 8 times num_kv_heads; hidden,
 * intermediate, target_hidden and num_q_heads*head_dim multiples of 64;
 * vocab a multiple of 16; FP8 weights with a bf16 dtype only.  Anything
 * else returns DFLASH_E_UNSUPPORTED. */
typedef struct {
  int32_t num_layers;        /* N_l draft layers */
  int32_t hidden;            /* D */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* d */
  int32_t intermediate;      /* I (SwiGLU) */
  int32_t vocab;             /* V */
  int32_t num_target_layers; /* n_t target layers fused per context row */
  int32_t target_hidden;     /* D_t */
  int32_t block_size;        /* K */
  int32_t mask_token_id;     /* id of the [MASK] token */
  int32_t dtype;             /* dflash_dtype */
  int32_t max_batch;         /* sequences (= KV-cache slots) */
  int32_t max_ctx;           /* max context length L per sequence */
  int32_t max_inject_rows;   /* max rows T per dflash_inject_kv call */
  float rope_theta;          /* RoPE base */
  float rms_eps;             /* RMSNorm epsilon */
  int32_t weight_format;     /* dflash_weight_format of the projections */
} dflash_config;

/* Drafter weights, PyTorch Linear layout [out, in], row-major, dtype of the
 * config (projections: see weight_format).  Per-layer entries are HOST
 * arrays of num_layers DEVICE pointers.  dflash_create copies every
 * projection matrix (fc, wq, wk, wv, wo, w_gate, w_up, w_down, lm_head) and
 * its scales into the context's own fragment-major layout and never reads
 * them again; embed and the norm gains are read in place and must stay
 * alive and unchanged until dflash_destroy.  The *_scale entries are read
 * only with FP8 weights ([out] fp32 each; 4-byte aligned) and are ignored
 * (may be NULL) otherwise. */
typedef struct {
  const void* embed;        /* [V, D] */
  const void* fc;           /* [D, n_t * D_t]: fuses the concatenated layers */
  const void* hidden_norm;  /* [D] RMSNorm gain applied after fc */
  const void* const* attn_norm;  /* [D]        per layer */
  const void* const* wq;         /* [Hq*d, D]  per layer */
  const void* const* wk;         /* [Hkv*d, D] per layer */
  const void* const* wv;         /* [Hkv*d, D] per layer */
  const void* const* wo;         /* [D, Hq*d]  per layer */
  const void* const* mlp_norm;   /* [D]        per layer */
  const void* const* w_gate;     /* [I, D]     per layer */
  const void* const* w_up;       /* [I, D]     per layer */
  const void* const* w_down;     /* [D, I]     per layer */
  const void* final_norm;   /* [D] */
  const void* lm_head;      /* [V, D] */
  const float* fc_scale;              /* [D] */
  const float* const* wq_scale;       /* [Hq*d]  per layer */
  const float* const* wk_scale;       /* [Hkv*d] per layer */
  const float* const* wv_scale;       /* [Hkv*d] per layer */
  const float* const* wo_scale;       /* [D]     per layer */
  const float* const* w_gate_scale;   /* [I]     per layer */
  const float* const* w_up_scale;     /* [I]     per layer */
  const float* const* w_down_scale;   /* [D]     per layer */
  const float* lm_head_scale;         /* [V] */
} dflash_weights;

typedef struct dflash_ctx dflash_ctx;

/* Create a drafting context on the current HIP device: validates the config
 * and weights, repacks the projection matrices (synchronises the device once),
 * and allocates the context's workspace (activations, attention and LM-head
 * partials, RoPE table, device error word).  *out is set on success. */
dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w,
                            dflash_ctx** out);

/* Free the context's workspace.  Waits for the device first.  NULL is a
 * no-op. */
void dflash_destroy(dflash_ctx* ctx);

/* Bytes of the KV cache for this config:
 *   num_layers * 2 * max_batch * num_kv_heads * (max_ctx + block_size)
 *   * head_dim * sizeof(dtype).
 * Layout kv[layer][0 = K | 1 = V][slot][kv_head][pos][head_dim].  Positions
 * [L, L + block_size) of a slot are scratch for the block being drafted. */
size_t dflash_kv_cache_bytes(const dflash_config* cfg);

/* Paged KV cache (serving-style storage of the context K/V; the pages'
 * method is unchanged, only where each position's K/V lives).
 *
 * dflash_set_kv_pages switches the context's cache addressing for the calls
 * that follow (inject, draft) from the contiguous layout above to pages:
 *   kv[layer][0 = K | 1 = V][page][kv_head][page_size][head_dim],
 * with position pos of slot s in page block_table[s * table_ld + pos /
 * page_size].  The cache then takes dflash_kv_cache_paged_bytes(cfg,
 * page_size, num_pages) bytes.
 *
 * page_size:   a power of two >= 64 (attention tiles of 64 keys never cross
 *              a page), or 0 to return to the contiguous layout.
 * num_pages:   pages per layer plane in the cache.
 * block_table: DEVICE int32 [max_batch][table_ld], owned by the caller and
 *              read by every later call (its contents may change between
 *              calls on the same stream).  Entries must exist for positions
 *              [0, L + block_size) of every slot drafted or injected; an id
 *              outside [0, num_pages) reads and writes page 0 and sets
 *              DFLASH_DEVERR_PAGE.
 * table_ld:    pages per slot; table_ld * page_size >= max_ctx + block_size.
 * Errors: DFLASH_E_INVALID (NULL ctx or table), DFLASH_E_SHAPE (sizes).
 * Results are identical to the contiguous layout's. */
dflash_status dflash_set_kv_pages(dflash_ctx* ctx, int32_t page_size,
                                  int32_t num_pages,
                                  const int32_t* block_table,
                                  int32_t table_ld);
/* num_layers * 2 * num_pages * num_kv_heads * page_size * head_dim
 * * sizeof(dtype); 0 for invalid arguments. */
size_t dflash_kv_cache_paged_bytes(const dflash_config* cfg, int32_t page_size,
                                   int32_t num_pages);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* dflash_last_error(void);

/* Test/debug only (synchronises `stream`): returns DFLASH_E_DEVICE and writes
 * the DFLASH_DEVERR_* bits to *bits if any were set since the last check,
 * then clears them.  bits may be NULL. */
dflash_status dflash_check_device_errors(dflash_ctx* ctx, void* stream,
                                         int32_t* bits);

/* Benchmark timing of one kernel class, on the stream it runs on.
 * kind: 0 = off, DFLASH_TIME_LMHEAD, DFLASH_TIME_ATTENTION (partial + merge),
 * DFLASH_TIME_GEMM (every projection GEMM launch, epilogues excluded).
 * While enabled, each launch of that class is bracketed by a pair of HIP
 * events created here (up to 8192 launches are kept; later ones overwrite
 * the oldest).  dflash_get_kernel_timing synchronises those events, returns
 * how many launches were recorded and their summed duration in
 * milliseconds, and clears the record.  Creating the events is the only
 * work set_kernel_timing does on the device. */
#define DFLASH_TIME_LMHEAD    1
#define DFLASH_TIME_ATTENTION 2
#define DFLASH_TIME_GEMM      3
dflash_status dflash_set_kernel_timing(dflash_ctx* ctx, int32_t kind);
dflash_status dflash_get_kernel_timing(dflash_ctx* ctx, int32_t* launches,
                                       double* total_ms);

/* KV injection of T context rows.
 *
 * Passage: "DFlash Guide", sections "2. Target Hidden-State Conditioning"
 * (H_cond = W_proj H_T) and "3. Cross-Layer KV Injection" (K^(l) = W_K^(l)
 * H_cond, V^(l) = W_V^(l) H_cond); sciencestack page, Figure 2 (features from
 * several target layers are fused and injected into every draft layer's KV
 * cache); stable-lab "KV Injection" (through the draft model's own K/V
 * projections, at every draft layer).
 *
 * For each row r < T:  c = RMSNorm(fc . concat_k target_hidden[k][r]) * g,
 * stored in the config dtype; then for every layer l and kv head h:
 *   kv[l][K][row_seq[r]][h][row_pos[r]][:] = RoPE(wk[l] . c, row_pos[r])
 *   kv[l][V][row_seq[r]][h][row_pos[r]][:] = wv[l] . c
 *
 * target_hidden: HOST array of num_target_layers DEVICE pointers, each to a
 *                [T, D_t] matrix with row stride `ld` elements (ld >= D_t).
 * row_seq, row_pos: [T] int32 slot in [0, max_batch) and position in
 *                [0, max_ctx).  Rows of one call must not repeat a
 *                (slot, pos) pair.
 * kv_cache:      dflash_kv_cache_bytes(cfg) bytes, written in place.
 * T:             1 <= T <= max_inject_rows.
 */
dflash_status dflash_inject_kv(dflash_ctx* ctx, void* stream,
                               const void* const* target_hidden, int64_t ld,
                               int32_t T, const int32_t* row_seq,
                               const int32_t* row_pos, void* kv_cache);

/* Draft one block per sequence in a single forward pass (or S passes).
 *
 * Passage: "DFlash Guide", section "1. Single-Pass Block-Diffusion Drafting"
 * (argmax over the drafter's output for a masked block given the context and
 * target features, one forward pass) and "Architectural Comparison" (the
 * block positions attend to each other bidirectionally); stable-lab "The
 * Model at a Glance" (S = 1-2 refinement passes committing positions in
 * confidence order; injected context is reused).
 *
 * Sequence b (slot b) has ctx_len[b] = L_b injected context positions.  The
 * block occupies positions L_b .. L_b+K-1; index 0 is the anchor (the last
 * verified token), indices 1..K-1 start as mask_token_id.  Each pass embeds
 * the block, runs every layer once over all K rows (attention over the L_b
 * context keys plus all K block keys, no mask), then the final norm and LM
 * head for still-masked rows only.  Per row: argmax (ties -> lowest id),
 * confidence = top-1 softmax probability, margin = top-1 minus top-2 logit.
 * Pass s < S commits the commit_per_pass most confident masked positions
 * (ties -> lower index); pass S commits the rest.
 *
 * batch:          1 <= batch <= max_batch.
 * anchor:         [batch] int32 anchor ids; ignored when block_tokens given.
 * block_tokens:   NULL, or [batch, K] int32 starting block: index 0 is the
 *                 anchor, mask_token_id marks masked positions, other ids
 *                 are already committed.
 * ctx_len:        [batch] int32 L_b in [0, max_ctx_len] (values outside
 *                 are clamped and set DFLASH_DEVERR_CTX_LEN).
 * max_ctx_len:    host upper bound on every ctx_len[b] (sizes the attention
 *                 grid), 0 <= max_ctx_len <= max_ctx.  A step captured in a
 *                 HIP graph keeps the grid of its capture: capture it with a
 *                 bound that covers every later ctx_len (e.g. max_ctx) when
 *                 the contexts grow between replays.  Results depend on the
 *                 bound only through float rounding (it sets how the keys
 *                 are split into chunks).
 * kv_cache:       as for dflash_inject_kv; positions [L_b, L_b+K) of each
 *                 slot are overwritten with the block's own K/V.
 * num_passes:     S >= 1; commit_per_pass c >= 1 when S > 1, with
 *                 c * (S-1) < K-1.
 * draft_tokens:   [batch, K-1] int32 out: the drafted id at block index i+1
 *                 (a position already committed in block_tokens is returned
 *                 as given).
 * confidence:     NULL or [batch, K-1] fp32 out (from the committing pass;
 *                 not written for positions committed in block_tokens).
 * top2_margin:    NULL or [batch, K-1] fp32 out (as confidence).
 * logits_debug:   NULL or [S, batch, K-1, V] fp32 out: logits of every row
 *                 computed in pass s (rows not computed are not written).
 *                 For parity tests only; costs a full logits write.
 */
dflash_status dflash_draft_block(dflash_ctx* ctx, void* stream, int32_t batch,
                                 const int32_t* anchor,
                                 const int32_t* block_tokens,
                                 const int32_t* ctx_len, int32_t max_ctx_len,
                                 void* kv_cache, int32_t num_passes,
                                 int32_t commit_per_pass,
                                 int32_t* draft_tokens, float* confidence,
                                 float* top2_margin, float* logits_debug);

/* Allocation-free variant of dflash_draft_block, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, same launch sequence,
 * same kernels and results, but the per-call scratch (activations,
 * attention and LM-head partials, the block state between passes, split-
 * contraction copies) comes from a static device buffer of
 * DFLASH_NOALLOC_SCRATCH_BYTES per GPU instead of the context's workspace.
 * The call allocates and frees nothing.
 *
 * The buffer is part of the library's code object: each GPU the library
 * runs on holds its own copy until the process ends.  Its device address is
 * resolved at dflash_create (with the context's device current).  Every call
 * on one GPU shares that GPU's buffer, and the buffer keeps the last call's
 * contents (nothing in it needs to start at zero), so calls that overlap on
 * one GPU -- on different streams, or through different contexts -- race:
 * order them.
 *
 * Scratch needed (256-byte aligned pieces, R = batch * K rows):
 *   R * D * 4 + 2 * R * D * esz + 2 * R * Hq*d * esz + R * I * esz
 *   + 3 * R * 4 + batch*(K-1) * (vocab/16 + 16) * 16
 *   + batch * Hq * nch * K * (d + 2) * 4 + 4 * R * D * 4
 * where esz is the dtype's size and nch the attention chunks per (sequence,
 * kv head) for this max_ctx_len; a call needing more than the buffer
 * returns DFLASH_E_CAPACITY and launches nothing.  With Qwen3-8B shapes
 * (D 4096, 32/8 heads of 128, I 12288, vocab 151936) a batch-1 call needs
 * about 9 MiB at a context of 2048, 19 MiB at 32768, and batch 4 at 32768
 * about 34 MiB. */
#define DFLASH_NOALLOC_SCRATCH_BYTES (64u << 20)
dflash_status dflash_draft_block_noalloc(
    dflash_ctx* ctx, void* stream, int32_t batch, const int32_t* anchor,
    const int32_t* block_tokens, const int32_t* ctx_len, int32_t max_ctx_len,
    void* kv_cache, int32_t num_passes, int32_t commit_per_pass,
    int32_t* draft_tokens, float* confidence, float* top2_margin,
    float* logits_debug);

/* Greedy verification.
 *
 * Passage: "DFlash Guide", section "The Cost Breakdown of Speculative Rounds"
 * (the target checks all drafts in one pass and keeps the longest valid
 * prefix; latency is amortised over tau + 1 tokens); stable-lab "Common
 * misconception" (nothing drafted survives unless the target agrees, so the
 * output is exactly the target's).  With greedy decoding the acceptance rule
 * is an exact match.
 *
 * draft_tokens:  [batch, K-1] int32, draft for block index j+1.
 * target_argmax: [batch, K] int32, the target's greedy id for block index
 *                j+1 (entry K-1 is the id after the last drafted position).
 * accept_len:    [batch] int32 out, tau + 1 where tau is the number of
 *                leading j with draft[j] == target[j] (1 <= accept_len <= K).
 * next_anchor:   [batch] int32 out, target_argmax[b][tau].
 * Needs no context; 1 <= block_size <= 64.
 */
dflash_status dflash_verify_greedy(void* stream, int32_t batch,
                                   int32_t block_size,
                                   const int32_t* draft_tokens,
                                   const int32_t* target_argmax,
                                   int32_t* accept_len, int32_t* next_anchor);

/* Speculative-sampling verification (sampled decoding, temperature > 0).
 *
 * Passage: "DFlash Guide", section "The Cost Breakdown of Speculative Rounds"
 * (the target keeps the longest valid prefix of the draft by rejection
 * sampling); stable-lab "Common misconception" (every drafted position must
 * clear the target's acceptance rule, so the output distribution is exactly
 * the target's).  The pages give no formula; this is the published rule of
 * speculative sampling (Leviathan, Kalman and Matias 2023; Chen et al. 2023):
 *   - drafted index j+1 with token x = draft_tokens[b][j] is accepted when
 *     u_accept[b][j] * q[b][j][x] < p[b][j][x], the product of the two
 *     float32 values taken exactly in float64; tau = the number of leading
 *     accepted positions;
 *   - if tau < K-1 the next token is drawn from the residual
 *     max(0, p[b][tau] - q[b][tau]) (float64 differences; from p[b][tau]
 *     itself when that residual is zero everywhere), else from p[b][K-1];
 *   - a draw takes the smallest index whose running float64 sum exceeds
 *     u_sample[b] times the total (never an index of weight zero).  The
 *     running sum adds 64-element tiles (each summed by a fixed pairwise
 *     tree) in index order, in segments of 64 tiles; at a boundary closer
 *     than rounding it can differ from a single sequential sum, and either
 *     index is a correct draw.  A distribution that is zero everywhere draws
 *     -1.
 * The drafter's own sampling (temperature, the draws that produced
 * draft_tokens) is the caller's: this call only judges a block.
 *
 * draft_tokens: [batch, K-1] int32; an id outside [0, vocab) is rejected.
 * draft_probs:  [batch, K-1, vocab] fp32 q, the draft distribution of each
 *               drafted index (rows need not be normalised exactly).
 * target_probs: [batch, K, vocab] fp32 p; row K-1 is the position after the
 *               block (the bonus token).  Entries must be finite and >= 0.
 * u_accept:     [batch, K-1] fp32 uniforms in [0, 1).
 * u_sample:     [batch] fp32 uniform in [0, 1).
 * accept_len:   [batch] int32 out, tau + 1 (1 <= accept_len <= K).
 * next_token:   [batch] int32 out, the drawn replacement or bonus token.
 * Needs no context; 2 <= block_size <= 64, 1 <= vocab <= 262144.  Reads at
 * most two vocabulary rows per sequence beyond the K-1 gathered
 * probabilities.
 */
dflash_status dflash_verify_sampling(void* stream, int32_t batch,
                                     int32_t block_size, int32_t vocab,
                                     const int32_t* draft_tokens,
                                     const float* draft_probs,
                                     const float* target_probs,
                                     const float* u_accept,
                                     const float* u_sample,
                                     int32_t* accept_len,
                                     int32_t* next_token);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
