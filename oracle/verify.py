"""Greedy and sampling verification, the synthetic target, and the pages'
accounting.

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


def sample_inverse_cdf(w, u):
    """Index drawn from the weights ``w`` (>= 0, not all zero) by inverse CDF
    at the uniform ``u`` in [0, 1): the smallest x whose running sum, taken in
    index order in float64, exceeds u times the total.  An index of weight 0
    is never returned."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    x = int(np.searchsorted(c, float(u) * c[-1], side="right"))
    return min(x, len(w) - 1)


def verify_sampling(draft, q, p, u_accept, u_sample):
    """Lossless speculative-sampling verification of one drafted block.

    The pages say the target accepts the longest valid prefix by rejection
    sampling, position by position, and that the output distribution stays
    the target's exactly ("DFlash Guide", section "The Cost Breakdown of
    Speculative Rounds"; stable-lab, "Common misconception").  They give no
    formula; this is the published rule of speculative sampling (Leviathan,
    Kalman and Matias 2023; Chen et al. 2023):

      * drafted index j (1..K-1, row j-1 here) with token x is accepted when
        u_j * q_j(x) < p_j(x), i.e. with probability min(1, p_j(x) / q_j(x));
        the product of the two float32 inputs is exact in float64;
      * at the first rejection the replacement token is drawn from the
        normalised residual max(0, p_j - q_j) (float64 differences); when that
        is zero everywhere, from p_j;
      * when every draft is accepted the bonus token is drawn from p_K.

    draft: [K-1] ids; q: [K-1, V] draft probabilities; p: [K, V] target
    probabilities (row K-1 is the position after the block); u_accept: [K-1]
    and u_sample: uniforms in [0, 1).  A drafted id outside [0, V) is
    rejected.  Returns (accept_len = tau + 1, next token).
    """
    draft = np.asarray(draft)
    q = np.asarray(q, dtype=np.float32)
    p = np.asarray(p, dtype=np.float32)
    k1, V = q.shape
    tau = 0
    while tau < k1:
        x = int(draft[tau])
        if not (0 <= x < V):
            break
        if float(np.float32(u_accept[tau])) * float(q[tau, x]) < float(p[tau, x]):
            tau += 1
        else:
            break
    if tau < k1:
        w = np.maximum(p[tau].astype(np.float64) - q[tau].astype(np.float64), 0.0)
        if not np.any(w > 0):
            w = p[tau].astype(np.float64)
    else:
        w = p[k1].astype(np.float64)
    return tau + 1, sample_inverse_cdf(w, np.float32(u_sample))


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
