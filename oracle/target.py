"""A small seeded target model and the speculative loop around the drafter
(oracle; test infrastructure).

The pages' loop: the target verifies a drafted block in one pass, keeps the
longest prefix it agrees with plus one token of its own, and the hidden
states it computed at several of its layers for the verified positions are
fused and injected into the drafter's cache before the next block ("DFlash
Guide", sections "The Cost Breakdown of Speculative Rounds" and "2. Target
Hidden-State Conditioning"; sciencestack page, Figure 2; stable-lab "The
Model at a Glance").  The target model itself is out of scope; this one is
a stand-in with the interface the loop needs:

  x_0 = E_t[token]                                  (the token's embedding)
  x_k = bf16(RMSNorm(x_{k-1} + W_k x_{k-1}) * g_k)  k = 1 .. n_t (hooks)
  z   = W_o x_{n_t};   greedy next token = argmax z (lowest id on ties)

Each position depends on its own token only (a bigram model: no attention),
so its features and its greedy token are the same whichever positions are
computed together.  The n_t hooked states x_1 .. x_{n_t} are the target
hidden states the drafter fuses.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from .numerics import rms_norm, round_bf16


def _f64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


class TargetModel:
    """Target weights (float64 copies of bf16 values)."""

    def __init__(self, tw: Dict[str, object]):
        self.E = _f64(tw["embed"])
        self.W = [_f64(t) for t in tw["layers"]]
        self.g = [_f64(t) for t in tw["gains"]]
        self.Wo = _f64(tw["head"])
        self.eps = float(tw.get("eps", 1e-6))


def target_forward(tm: TargetModel, tokens: Sequence[int]):
    """Hooked hidden states [n_t][rows, D_t] (bf16 values), the greedy next
    token per row, and its top-2 logit margin."""
    x = tm.E[np.asarray(tokens, dtype=np.int64)]
    hooks = []
    for W, g in zip(tm.W, tm.g):
        x = round_bf16(rms_norm(x + x @ W.T, g, tm.eps))
        hooks.append(x)
    z = x @ tm.Wo.T
    nxt = np.argmax(z, axis=1)
    srt = np.sort(z, axis=1)
    return hooks, nxt.astype(np.int64), srt[:, -1] - srt[:, -2]


def greedy_stream(tm: TargetModel, start: int, n: int) -> List[int]:
    """The target's own greedy continuation of `start`: n tokens."""
    out, t = [], int(start)
    for _ in range(n):
        t = int(target_forward(tm, [t])[1][0])
        out.append(t)
    return out


def speculative_loop(model, tm: TargetModel, prompt: Sequence[int],
                     n_emit: int, drafts_from_target=None):
    """Draft -> verify -> capture -> inject rounds for one sequence.

    The prompt's hooked target states are injected first (positions
    0 .. L0-1) and the anchor is the target's greedy token after the prompt.
    Each round drafts a block after the L verified tokens, the target
    verifies the block [anchor, d_1 .. d_15] in one pass (its greedy token
    after every block position), the accepted prefix plus the anchor is
    appended, and the target's hooked states of those accepted positions --
    computed in the verify pass -- are injected at positions L .. L+a-1.
    drafts_from_target(round) optionally gives how many leading drafts to
    replace by the target's own continuation (a drafter that is right for
    a while).  Returns (emitted stream, accept lengths per round)."""
    from .drafter import draft_batch, inject_rows
    from .verify import verify_greedy
    K = model.K
    prompt = [int(t) for t in prompt]
    hooks, nxt, _ = target_forward(tm, prompt)
    ctx = inject_rows(model, hooks, np.arange(len(prompt)))
    y, anchor, accepts = list(prompt), int(nxt[-1]), []
    r = 0
    while len(y) < len(prompt) + n_emit:
        L = len(y)
        d = list(draft_batch(model, [ctx], [L], anchors=[anchor])[0]["draft"])
        if drafts_from_target is not None:
            c = int(drafts_from_target(r))
            chain = greedy_stream(tm, anchor, c)
            d[:c] = chain
        block = [anchor] + [int(t) for t in d]
        hooks_b, nxt_b, _ = target_forward(tm, block)
        acc, anchor = verify_greedy(d, nxt_b)
        new = inject_rows(model, [h[:acc] for h in hooks_b],
                          np.arange(L, L + acc))
        ctx = {l: (np.concatenate([ctx[l][0], new[l][0]]),
                   np.concatenate([ctx[l][1], new[l][1]])) for l in ctx}
        y += block[:acc]
        accepts.append(acc)
        r += 1
    return y, accepts
