"""Greedy verification, the synthetic target, and the pages' accounting.

Oracle / test infrastructure.  Sources:
  * acceptance of the longest matching prefix plus one token from the target,
    and the latency-per-token formula: "DFlash Guide", section "The Cost
    Breakdown of Speculative Rounds";
  * losslessness of the acceptance rule: "DFlash Guide", "Key Takeaways";
    stable-lab, "Common misconception";
  * the toy drafting race, cycle (K+12) ticks against (S+12): stable-lab,
    "Watch the Block Get Drafted".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence

import numpy as np


def verify_greedy(draft, target):
    """Accept the longest prefix of the draft that the target agrees with.

    draft: [K-1] drafted ids for block indices 1..K-1.
    target: [K] the target's greedy id for block indices 1..K (index K is
    the token after the last drafted position).
    tau = largest n with draft[j] == target[j] for all j < n; the accepted
    length is tau + 1 (tau drafts plus the target's own token at tau), and
    that token target[tau] is the next block's anchor.  With greedy decoding
    the page's rejection-sampling rule reduces to this exact-match rule.
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    tau = 0
    while tau < len(draft) and draft[tau] == target[tau]:
        tau += 1
    return tau + 1, int(target[tau])


def synthetic_target(draft, u, r, tail, p, vocab):
    """Stand-in for the target model's greedy ids (harness, not the method).

    For drafted index j: the target agrees with the draft when u[j] < p[j];
    otherwise it picks (draft[j] + 1 + r[j]) mod V, which never equals the
    draft.  The last slot (after the block) is ``tail``.
    draft/u/r: [B, K-1]; tail: [B]; p: [K-1].  Returns [B, K] int64.
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, k1 = draft.shape
    T = np.empty((B, k1 + 1), dtype=np.int64)
    agree = np.asarray(u, dtype=np.float32) < np.asarray(p, dtype=np.float32)
    T[:, :k1] = np.where(agree, draft,
                         (draft + 1 + np.asarray(r, dtype=np.int64)) % vocab)
    T[:, k1] = np.asarray(tail, dtype=np.int64)
    return T


def expected_accept_len(p: Sequence[float]):
    """E[tau + 1] when drafted index j matches independently with prob p[j]:
    1 + sum_n prod_{j <= n} p[j]."""
    total, run = 1.0, 1.0
    for pj in p:
        run *= pj
        total += run
    return total


def latency_per_token(t_draft, t_verify, tau):
    """(T_draft + T_verify) / (tau + 1); T_draft = gamma * t_step for an
    autoregressive drafter, S * t_pass for the block drafter."""
    return Fraction(t_draft + t_verify) / (tau + 1)


def simulate_rounds(draft_passes, t_pass, t_verify, taus):
    """Tick-level event simulation of speculative rounds.

    Each round runs ``draft_passes`` draft passes of ``t_pass`` ticks, one
    verify pass of ``t_verify`` ticks, then emits tau + 1 tokens.  Returns the
    per-round latency per token (ticks / tokens) and the overall one.
    """
    clock = 0
    per_round, emitted = [], 0
    for tau in taus:
        start = clock
        for _ in range(draft_passes):
            for _ in range(t_pass):
                clock += 1
        for _ in range(t_verify):
            clock += 1
        emitted += tau + 1
        per_round.append(Fraction(clock - start, tau + 1))
    return per_round, Fraction(clock, emitted)


def simulate_toy_race(K, S, verify_ticks=12, cycles=50, alpha=0.7, seed=0):
    """The toy race: both lanes draft the same K-block and face the same
    acceptance coins, so they accept identical tokens; the autoregressive
    lane spends one tick per drafted token, the block lane one tick per
    refinement pass.  Returns (ticks_ar, ticks_block, accepted, ratio)."""
    rng = np.random.default_rng(seed)
    ticks_ar = ticks_blk = 0
    accepted = 0
    for _ in range(cycles):
        coins = rng.random(K) < alpha
        tau = 0
        while tau < K and coins[tau]:
            tau += 1
        for _ in range(K):
            ticks_ar += 1
        for _ in range(S):
            ticks_blk += 1
        ticks_ar += verify_ticks
        ticks_blk += verify_ticks
        accepted += tau + 1
    return ticks_ar, ticks_blk, accepted, Fraction(ticks_ar, ticks_blk)


def toy_race_ratio(K, S, verify_ticks=12):
    """(K + verify) / (S + verify): the block lane's speed edge per cycle."""
    return Fraction(K + verify_ticks, S + verify_ticks)
