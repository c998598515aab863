"""The DFlash drafter, step by step, in float64 (oracle; test infrastructure).

Order and notation follow the pages:
  * target hidden states H_T from several target layers are fused into
    H_cond by one projection ("DFlash Guide", section "2. Target Hidden-State
    Conditioning"; fused per the sciencestack page, Figure 2);
  * every draft layer l injects K^(l) = W_K^(l) H_cond, V^(l) = W_V^(l) H_cond
    into its own KV cache ("DFlash Guide", "3. Cross-Layer KV Injection";
    stable-lab "DFlash: Diffusion Drafts the Block", "KV Injection");
  * a block of gamma = K positions is drafted by ONE forward pass of the
    drafter D_theta over masked positions ("DFlash Guide", "1. Single-Pass
    Block-Diffusion Drafting", the argmax equation), with bidirectional
    attention among block positions ("DFlash Guide", "Architectural
    Comparison"), optionally repeated for S refinement passes that commit
    positions in confidence order (stable-lab, "The Model at a Glance").

Readings taken where the pages are silent:
block = [anchor, m, ..., m] with the anchor the last verified token, drafts at
block indices 1..K-1; fusion = concat of the n_t layers in caller order -> fc
-> RMSNorm with gain; no norm between H_cond and the K/V projections; RoPE on
K only; pre-norm decoder layers without biases; SwiGLU; no attention mask;
scale 1/sqrt(d); GQA group h // (Hq/Hkv); argmax ties -> lowest id; commit
ties -> lowest block index; bf16 storage rounding at the points the bf16
drafter stores tensors, float64 everywhere else.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .numerics import (dequant_rows, identity_round, logsumexp, rms_norm,
                       rope, round_bf16, silu, softmax)


def _f64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    import torch  # weights may arrive as torch tensors from the generators
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _f32(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float32)
    import torch
    return t.detach().to("cpu", torch.float32).numpy()


def _codes(t):
    """Raw bytes of an FP8 weight tensor (torch float8 or uint8)."""
    import torch
    t = t.detach().to("cpu")
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    return t.numpy()


def _weight(weights, key, l=None):
    """A projection matrix as float64: given in the drafter dtype, or as
    FP8 E4M3 codes with a per-output-row scale (key + "_scale")."""
    t = weights[key] if l is None else weights[key][l]
    sk = key + "_scale"
    if sk in weights and weights[sk] is not None:
        sc = weights[sk] if l is None else weights[sk][l]
        return dequant_rows(_codes(t), _f64(sc))
    return _f64(t)


class OracleModel:
    """Drafter weights on the host plus the shape they belong to.

    Per-layer matrices are kept in float64.  The two vocabulary-sized
    matrices (embedding, LM head) are kept in float32, which holds bf16 and
    f32 values exactly, and are widened to float64 a slice at a time.
    """

    def __init__(self, wl, weights, layers: Optional[Sequence[int]] = None):
        self.wl = wl
        self.rnd = round_bf16 if wl.dtype == "bf16" else identity_round
        self.D, self.Hq, self.Hkv, self.d = (wl.hidden, wl.num_q_heads,
                                             wl.num_kv_heads, wl.head_dim)
        self.theta, self.eps, self.K = wl.rope_theta, wl.rms_eps, wl.block_size
        self.mask_id = wl.mask_id
        self.E = _f32(weights["embed"])
        # the LM head is widened to float64 a slice at a time (lm_rows): kept
        # in float32 (exact for bf16 / f32 values) or, FP8, as its codes and
        # per-row scales
        if weights.get("lm_head_scale") is not None:
            self.W_lm = None
            self.lm_codes = _codes(weights["lm_head"])
            self.lm_scale = _f64(weights["lm_head_scale"])
        else:
            self.W_lm = _f32(weights["lm_head"])
        self.W_fc = _weight(weights, "fc")
        self.g_h = _f64(weights["hidden_norm"])
        self.g_f = _f64(weights["final_norm"])
        n = wl.num_layers
        self.layers = list(range(n)) if layers is None else list(layers)
        self.L = {}
        for l in self.layers:
            self.L[l] = {k: _f64(weights[k][l]) for k in (
                "attn_norm", "mlp_norm")}
            self.L[l].update({k: _weight(weights, k, l) for k in (
                "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")})
        self.layer_calls = 0  # decoder-layer invocations (single-pass check)

    @property
    def vocab(self) -> int:
        return (self.W_lm if self.W_lm is not None else self.lm_codes).shape[0]

    def lm_rows(self, c0: int, c1: int):
        """LM-head rows [c0, c1) in float64."""
        if self.W_lm is not None:
            return self.W_lm[c0:c1].astype(np.float64)
        return dequant_rows(self.lm_codes[c0:c1], self.lm_scale[c0:c1])


# ---------------------------------------------------------------------------
# a1 + a2: fusion and KV injection
# ---------------------------------------------------------------------------

def fuse_features(H_T: Sequence[np.ndarray], W_proj, g, eps, rnd):
    """H_cond = RMSNorm(W_proj . concat(H_T^1 .. H_T^n_t)) per context row.

    "DFlash Guide", section 2 (H_cond = W_proj H_T); several target layers
    are fused (sciencestack page, Figure 2).  The n_t layers are concatenated
    along features in the order given.
    """
    f = np.concatenate([_f64(h) for h in H_T], axis=1)      # [T, n_t*D_t]
    u = f @ W_proj.T                                        # [T, D]
    return rnd(rms_norm(u, g, eps))


def inject_kv(H_cond, W_K, W_V, pos, theta, n_kv, d, rnd):
    """K^(l) = RoPE(W_K^(l) H_cond), V^(l) = W_V^(l) H_cond for one layer.

    "DFlash Guide", section 3 (the K_draft/V_draft equation); stable-lab
    "KV Injection" (target representations pass through the draft model's
    own KV projections into its cache).  Returns [T, Hkv, d] each.
    """
    T = H_cond.shape[0]
    k = (H_cond @ W_K.T).reshape(T, n_kv, d)
    v = (H_cond @ W_V.T).reshape(T, n_kv, d)
    return rnd(rope(k, pos, theta)), rnd(v)


def inject_rows(model: OracleModel, H_T, pos) -> Dict[int, tuple]:
    """Fuse once, inject into every draft layer: {layer: (K, V)}."""
    c = fuse_features(H_T, model.W_fc, model.g_h, model.eps, model.rnd)
    out = {}
    for l in model.layers:
        P = model.L[l]
        out[l] = inject_kv(c, P["wk"], P["wv"], np.asarray(pos), model.theta,
                           model.Hkv, model.d, model.rnd)
    return out


# ---------------------------------------------------------------------------
# a3 .. a8: one drafter pass over the block
# ---------------------------------------------------------------------------

def block_attention(q, keys, vals):
    """Softmax attention of block queries over all keys, no mask.

    q: [K, Hq, d]; keys/vals: [L + K, Hkv, d] (injected context, then the
    block's own keys).  Every block query sees every key: the block is
    bidirectional ("DFlash Guide", "Architectural Comparison") and the
    context is fully visible.  Query head h reads kv head h // (Hq/Hkv).
    """
    Kq, Hq, d = q.shape
    Hkv = keys.shape[1]
    group = Hq // Hkv
    o = np.empty_like(q)
    for h in range(Hq):
        kh = h // group
        s = q[:, h, :] @ keys[:, kh, :].T / np.sqrt(d)      # [K, L+K]
        o[:, h, :] = softmax(s, axis=-1) @ vals[:, kh, :]
    return o


def decoder_layer(model: OracleModel, l: int, x, ctx_k, ctx_v, pos):
    """One pre-norm drafter layer over the K block rows (residual x, f64)."""
    P, r = model.L[l], model.rnd
    Kb = x.shape[0]
    model.layer_calls += 1
    h = r(rms_norm(x, P["attn_norm"], model.eps))
    q = r(rope((h @ P["wq"].T).reshape(Kb, model.Hq, model.d), pos,
               model.theta))
    k = r(rope((h @ P["wk"].T).reshape(Kb, model.Hkv, model.d), pos,
               model.theta))
    v = r((h @ P["wv"].T).reshape(Kb, model.Hkv, model.d))
    keys = np.concatenate([ctx_k, k], axis=0)
    vals = np.concatenate([ctx_v, v], axis=0)
    o = r(block_attention(q, keys, vals)).reshape(Kb, model.Hq * model.d)
    x = x + o @ P["wo"].T
    h2 = r(rms_norm(x, P["mlp_norm"], model.eps))
    a = r(silu(h2 @ P["w_gate"].T) * (h2 @ P["w_up"].T))
    return x + a @ P["w_down"].T


def lm_logits(model: OracleModel, x_rows, chunk: int = 16384):
    """z = W_lm . RMSNorm(x; g_f) in float64, never rounded."""
    hf = model.rnd(rms_norm(x_rows, model.g_f, model.eps))
    V = model.vocab
    z = np.empty((hf.shape[0], V), dtype=np.float64)
    for c0 in range(0, V, chunk):
        z[:, c0:c0 + chunk] = hf @ model.lm_rows(c0, c0 + chunk).T
    return z


def lm_head_reduce(z):
    """Per row: argmax (lowest id on ties), top-1, top-2, log-sum-exp,
    confidence = top-1 softmax probability, margin = top1 - top2.

    The argmax is the drafted token ("DFlash Guide", section 1, argmax over
    D_theta); the confidence is what the S-pass commit orders by
    (stable-lab, "The Model at a Glance").
    """
    z = np.atleast_2d(np.asarray(z, dtype=np.float64))
    tok = np.argmax(z, axis=1)                        # first max = lowest id
    srt = np.sort(z, axis=1)
    top1, top2 = srt[:, -1], srt[:, -2]
    lse = logsumexp(z, axis=1)
    return {"token": tok.astype(np.int64), "top1": top1, "top2": top2,
            "lse": lse, "conf": np.exp(top1 - lse), "margin": top1 - top2}


def confidence_commit(conf, masked, count: Optional[int]):
    """Block indices to commit this pass.

    Among still-masked positions, the ``count`` most confident, ties to the
    lower block index; ``count=None`` commits every masked position (the last
    pass).  Confidence order per stable-lab, "The Model at a Glance".
    """
    idx = [i for i in range(len(masked)) if masked[i]]
    if count is None or count >= len(idx):
        return sorted(idx)
    ranked = sorted(idx, key=lambda i: (-conf[i], i))
    return sorted(ranked[:count])


def draft_sequence(model: OracleModel, ctx_kv: Dict[int, tuple], L: int,
                   tokens, committed, num_passes: int = 1,
                   commit_per_pass: int = 0, keep_logits: bool = False):
    """Draft one sequence's block.

    ctx_kv: {layer: (K [L, Hkv, d], V [L, Hkv, d])} -- injected context.
    tokens/committed: [K] block ids and which are fixed; index 0 (anchor)
    must be committed.  Pass s embeds the current block (masks, anchor and
    committed ids), runs every layer once over all K positions at positions
    L..L+K-1, takes logits for still-masked positions only and commits
    ``commit_per_pass`` of them by confidence (all of them in the last pass).
    Injected KV is reused by every pass; nothing is re-injected.
    """
    K = model.K
    tokens = np.array(tokens, dtype=np.int64).copy()
    committed = np.array(committed, dtype=bool).copy()
    assert committed[0]
    pos = L + np.arange(K)
    res = {"conf": np.full(K, np.nan), "margin": np.full(K, np.nan),
           "lse": np.full(K, np.nan), "pass": np.full(K, -1),
           "logits": [], "pass_conf": [], "masked_rows": []}
    for s in range(num_passes):
        masked = ~committed
        x = model.E[tokens].astype(np.float64)                 # [K, D]
        for l in model.layers:
            x = decoder_layer(model, l, x, ctx_kv[l][0], ctx_kv[l][1], pos)
        rows = np.nonzero(masked)[0]
        z = lm_logits(model, x[rows])
        red = lm_head_reduce(z)
        conf = np.full(K, np.nan)
        conf[rows] = red["conf"]
        last = s == num_passes - 1
        chosen = confidence_commit(conf, masked, None if last
                                   else commit_per_pass)
        where = {int(i): j for j, i in enumerate(rows)}
        for i in chosen:
            j = where[i]
            tokens[i] = red["token"][j]
            committed[i] = True
            res["conf"][i] = red["conf"][j]
            res["margin"][i] = red["margin"][j]
            res["lse"][i] = red["lse"][j]
            res["pass"][i] = s
        res["masked_rows"].append(rows)
        res["pass_conf"].append(conf)
        res["logits"].append(z if keep_logits else None)
        res.setdefault("pass_margin", []).append(
            dict(zip(rows.tolist(), red["margin"].tolist())))
        res.setdefault("pass_token", []).append(
            dict(zip(rows.tolist(), red["token"].tolist())))
    res["tokens"] = tokens
    res["draft"] = tokens[1:]
    return res


def draft_batch(model: OracleModel, ctx_kv_per_seq: List[Dict[int, tuple]],
                ctx_len, anchors=None, block_tokens=None, num_passes=1,
                commit_per_pass=0, keep_logits=False, seqs=None):
    """draft_sequence for each sequence b (independent of one another).

    Either ``anchors`` [B] (block = anchor then K-1 masks) or
    ``block_tokens`` [B, K] (mask id = still masked; index 0 is the anchor).
    ``seqs`` restricts the work to some sequences; ``ctx_kv_per_seq`` is
    indexed like ``seqs``.
    """
    K, m = model.K, model.mask_id
    B = len(ctx_len)
    seqs = list(range(B)) if seqs is None else list(seqs)
    out = []
    for j, b in enumerate(seqs):
        if block_tokens is not None:
            tok = np.array(block_tokens[b], dtype=np.int64)
            com = tok != m
            com[0] = True
        else:
            tok = np.full(K, m, dtype=np.int64)
            tok[0] = int(anchors[b])
            com = np.zeros(K, dtype=bool)
            com[0] = True
        out.append(draft_sequence(model, ctx_kv_per_seq[j], int(ctx_len[b]),
                                  tok, com, num_passes, commit_per_pass,
                                  keep_logits))
    return out
