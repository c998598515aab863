"""How far an exact float32 evaluation of the drafting pass lands from the
float64 oracle: the floor under the logit tolerance of any implementation
that accumulates in float32 and stores activations in bf16.

The pass is evaluated once more with torch float32 arithmetic on the CPU,
rounding to bf16 (correctly, with the oracle's rounding) at exactly the
oracle's storage points: norm outputs, q/k/v after RoPE, the attention
output, SiLU(gate)*up and the final-norm rows.  No GPU code is involved.
The float32 evaluation is as correct as float32 allows, yet its bf16
roundings disagree with the float64 ones on a few elements per row, and each
disagreement moves the next normalisation of the residual stream for every
element of the row; the MLP spreads the resulting rounding flips over the
whole hidden state.  Measured at Qwen3-8B shapes (context 2048, vocabulary
151936): max |logit difference| 1.77e-2 (1 draft layer), 3.36e-2 (3 layers),
4.46e-2 (5 layers).

Usage: python -m tests.precision_floor [--layers 1 3 5] [--vocab 151936]
(CPU, about a minute per layer count; not collected by pytest).
"""
from __future__ import annotations

import argparse

import numpy as np
import torch

import workloads as W
from oracle import OracleModel, draft_batch
from oracle.numerics import round_bf16


def _bf16(t: torch.Tensor) -> torch.Tensor:
    return torch.from_numpy(round_bf16(t.double().numpy())).float()


def _rms(x, g, eps):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g


def _rope(x, pos, theta):
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2 / d)
    ang = pos[:, None].double() * inv[None, :]
    c = torch.cos(ang).float()[:, None, :]
    s = torch.sin(ang).float()[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * c - b * s, b * c + a * s], -1)


def float32_pass(wl, w, prefix, anchor, L):
    """Logits of the 15 masked rows, float32 arithmetic, bf16 storage."""
    f = lambda t: t.to(torch.float32)
    K, Hq, Hkv, d = wl.block_size, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    eps, theta = wl.rms_eps, wl.rope_theta
    tok = torch.full((K,), wl.mask_id)
    tok[0] = anchor
    x = f(w["embed"][tok])
    pos = torch.arange(L, L + K)
    for l in range(wl.num_layers):
        h = _bf16(_rms(x, f(w["attn_norm"][l]), eps))
        q = _bf16(_rope((h @ f(w["wq"][l]).T).view(K, Hq, d), pos, theta))
        k = _bf16(_rope((h @ f(w["wk"][l]).T).view(K, Hkv, d), pos, theta))
        v = _bf16((h @ f(w["wv"][l]).T).view(K, Hkv, d))
        keys = torch.cat([f(prefix[l][0]).transpose(0, 1), k], 0)
        vals = torch.cat([f(prefix[l][1]).transpose(0, 1), v], 0)
        o = torch.empty(K, Hq, d)
        for hh in range(Hq):
            kh = hh // (Hq // Hkv)
            s = q[:, hh] @ keys[:, kh].T / (d ** 0.5)
            o[:, hh] = torch.softmax(s, -1) @ vals[:, kh]
        o = _bf16(o.reshape(K, Hq * d))
        x = x + o @ f(w["wo"][l]).T
        h2 = _bf16(_rms(x, f(w["mlp_norm"][l]), eps))
        a = _bf16(torch.nn.functional.silu(h2 @ f(w["w_gate"][l]).T) *
                  (h2 @ f(w["w_up"][l]).T))
        x = x + a @ f(w["w_down"][l]).T
    hf = _bf16(_rms(x[1:], f(w["final_norm"]), eps))
    return (hf @ f(w["lm_head"]).T).double().numpy()


def floor(num_layers: int, vocab: int = 151936, L: int = 2048):
    wl = W.WORKLOADS["qwen3-8b-1L-b1-ctx2048"].replace(num_layers=num_layers,
                                                       vocab=vocab)
    w = W.gen_weights(wl)
    prefix = {l: (W.gen_kv_prefix(wl, l, "k", 0, L),
                  W.gen_kv_prefix(wl, l, "v", 0, L)) for l in range(num_layers)}
    anchor = int(W.gen_anchors(wl)[0])
    z32 = float32_pass(wl, w, prefix, anchor, L)
    model = OracleModel(wl, w)
    ctx = {l: (W.to_f64(prefix[l][0]).transpose(1, 0, 2),
               W.to_f64(prefix[l][1]).transpose(1, 0, 2))
           for l in range(num_layers)}
    z64 = draft_batch(model, [ctx], [L], anchors=[anchor],
                      keep_logits=True)[0]["logits"][0]
    dz = np.abs(z32 - z64)
    return float(dz.max()), float(dz.mean()), float(z64.std())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, nargs="+", default=[1, 3, 5])
    ap.add_argument("--vocab", type=int, default=151936)
    args = ap.parse_args()
    torch.set_num_threads(8)
    for n in args.layers:
        mx, mean, sig = floor(n, args.vocab)
        print(f"{n} draft layer(s): max |dz| {mx:.3e}, mean {mean:.2e}, "
              f"logit std {sig:.3f}", flush=True)


if __name__ == "__main__":
    main()
