"""A second evaluation of the drafting step, composed from torch library ops
(test helper; no GPU code, no oracle code but the pinned bf16 rounding).

It computes what the oracle computes -- fusion, injection into every layer,
the pre-norm layers over the block, final norm and LM head -- with the bf16
storage rounding at the same points (H_cond, injected K and V, every norm
output, q/k after RoPE, v, the attention output, SiLU(gate)*up), in either
of two arithmetics:

  * float64: then it must reproduce the oracle to rounding of float64 sums
    (the bf16 roundings agree unless a value falls within ~1e-16 of a
    rounding midpoint).  This pins the oracle's rounding placement against
    an independent composition.
  * float32: any correct implementation that accumulates in float32 and
    stores bf16 lands about this far from the float64 oracle.  Each bf16
    rounding that the float32 sums decide differently moves whole rows of
    the next projection, and the following norm and MLP spread those moves
    over the hidden state, so the distance grows with depth.  ``member`` >
    0 sums every projection's contraction in chunks in a seeded order, a
    different but equally correct float32 evaluation; an ensemble of them
    samples how far, and on which tokens, float32 arithmetic can land from
    the oracle.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch
import torch.nn.functional as F

from oracle.numerics import round_bf16  # pinned exhaustively on its own


class Prepared:
    """Weights of one workload converted once to the evaluation dtype."""

    def __init__(self, wl, w: Dict[str, object], dtype=torch.float32,
                 layers: Optional[Sequence[int]] = None):
        self.wl, self.dtype = wl, dtype
        cv = lambda t: t.detach().to("cpu").to(dtype)

        def mat(key, l=None):
            # a projection: (matrix, per-row scale or None); FP8 codes are
            # widened exactly and their scale applied after the product
            t = w[key] if l is None else w[key][l]
            sc = w.get(key + "_scale")
            if sc is not None:
                sc = cv(sc if l is None else sc[l])
            return (cv(t), sc)

        self.embed = w["embed"]  # gathered by row, converted per pass
        self.fc = mat("fc")
        self.hidden_norm = cv(w["hidden_norm"])
        self.final_norm = cv(w["final_norm"])
        self.lm_head = mat("lm_head")
        self.layers = list(range(wl.num_layers)) if layers is None else list(
            layers)
        self.L = {l: dict({k: cv(w[k][l]) for k in ("attn_norm",
                                                      "mlp_norm")},
                          **{k: mat(k, l) for k in (
                              "wq", "wk", "wv", "wo", "w_gate", "w_up",
                              "w_down")})
                  for l in self.layers}


def _store(p: Prepared, t: torch.Tensor) -> torch.Tensor:
    """bf16 storage point (identity for an f32 drafter)."""
    if p.wl.dtype != "bf16":
        return t
    r = round_bf16(t.detach().to(torch.float64).numpy())
    return torch.from_numpy(r).to(p.dtype)


def _linear(p: Prepared, x: torch.Tensor, Ws, member: int,
            tag: int) -> torch.Tensor:
    """x . W^T in the evaluation dtype (times the per-row scale of FP8
    weights); member > 0 sums the contraction in seeded chunks in a seeded
    order."""
    W, sc = Ws
    y = _product(x, W, member, tag)
    return y if sc is None else y * sc


def _product(x, W, member, tag):
    if member == 0:
        return F.linear(x, W)
    Kd = W.shape[1]
    rng = np.random.default_rng([member, tag, Kd])
    chunk = int(rng.choice([32, 64, 128, 256, 512]))
    chunk = min(chunk, Kd)
    starts = list(range(0, Kd, chunk))
    rng.shuffle(starts)
    acc = None
    for s in starts:
        part = F.linear(x[..., s:s + chunk], W[:, s:s + chunk])
        acc = part if acc is None else acc + part
    return acc


def _rope(x: torch.Tensor, pos: np.ndarray, theta: float) -> torch.Tensor:
    """Rotate-half RoPE; angles in float64, then the evaluation dtype."""
    d = x.shape[-1]
    inv = theta ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = torch.from_numpy(np.cos(ang)).to(x.dtype)[:, None, :]
    s = torch.from_numpy(np.sin(ang)).to(x.dtype)[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def _rms(p: Prepared, x: torch.Tensor, g: torch.Tensor) -> torch.Tensor:
    return F.rms_norm(x, (x.shape[-1],), weight=g, eps=p.wl.rms_eps)


def inject(p: Prepared, hiddens: Sequence[torch.Tensor], pos,
           member: int = 0) -> Dict[int, tuple]:
    """{layer: (K [T, Hkv, d], V [T, Hkv, d])} float64 arrays."""
    wl = p.wl
    f = torch.cat([h.detach().to("cpu").to(p.dtype) for h in hiddens], 1)
    c = _store(p, _rms(p, _linear(p, f, p.fc, member, 1), p.hidden_norm))
    T = c.shape[0]
    out = {}
    for l in p.layers:
        P = p.L[l]
        k = _linear(p, c, P["wk"], member, 10 + l).reshape(
            T, wl.num_kv_heads, wl.head_dim)
        v = _linear(p, c, P["wv"], member, 20 + l).reshape(
            T, wl.num_kv_heads, wl.head_dim)
        out[l] = (_store(p, _rope(k, pos, wl.rope_theta)).double().numpy(),
                  _store(p, v).double().numpy())
    return out


def _attention(q, keys, vals):
    """Non-causal softmax attention, GQA by repeating kv heads."""
    group = q.shape[1] // keys.shape[1]
    qt = q.permute(1, 0, 2)
    kt = keys.repeat_interleave(group, 1).permute(1, 0, 2)
    vt = vals.repeat_interleave(group, 1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=False)
    return o.permute(1, 0, 2)


def pass_logits(p: Prepared, ctx_kv: Dict[int, tuple], L: int,
                block_tokens: Sequence[int], member: int = 0):
    """One pass over the block [K] (mask id = still masked): returns
    (masked block indices, logits [rows, V] float64 numpy)."""
    wl = p.wl
    K, Hq, Hkv, d = wl.block_size, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    tok = torch.as_tensor(np.asarray(block_tokens, dtype=np.int64))
    x = p.embed[tok].to("cpu").to(p.dtype)
    pos = np.arange(L, L + K)
    for l in p.layers:
        P = p.L[l]
        h = _store(p, _rms(p, x, P["attn_norm"]))
        q = _linear(p, h, P["wq"], member, 100 + l).reshape(K, Hq, d)
        k = _linear(p, h, P["wk"], member, 200 + l).reshape(K, Hkv, d)
        v = _linear(p, h, P["wv"], member, 300 + l).reshape(K, Hkv, d)
        q = _store(p, _rope(q, pos, wl.rope_theta))
        k = _store(p, _rope(k, pos, wl.rope_theta))
        v = _store(p, v)
        keys = torch.cat([torch.as_tensor(ctx_kv[l][0]).to(p.dtype), k], 0)
        vals = torch.cat([torch.as_tensor(ctx_kv[l][1]).to(p.dtype), v], 0)
        o = _store(p, _attention(q, keys, vals).reshape(K, Hq * d))
        x = x + _linear(p, o, P["wo"], member, 400 + l)
        h2 = _store(p, _rms(p, x, P["mlp_norm"]))
        a = _store(p, F.silu(_linear(p, h2, P["w_gate"], member, 500 + l)) *
                   _linear(p, h2, P["w_up"], member, 600 + l))
        x = x + _linear(p, a, P["w_down"], member, 700 + l)
    rows = np.array([i for i in range(1, K) if block_tokens[i] == wl.mask_id],
                    dtype=np.int64)
    hf = _store(p, _rms(p, x[rows], p.final_norm))
    return rows, _linear(p, hf, p.lm_head, member, 9).double().numpy()
