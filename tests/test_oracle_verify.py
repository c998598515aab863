"""Pins for greedy verification, the synthetic target and the pages'
accounting formulas.  CPU only."""
import hashlib
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import (expected_accept_len, latency_per_token, simulate_rounds,
                    simulate_toy_race, synthetic_target, toy_race_ratio,
                    verify_greedy)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_verify_exhaustive_all_match_patterns():
    # every one of the 2^15 match patterns of a K = 16 block
    K1 = 15
    rng = np.random.default_rng(0)
    draft = rng.integers(0, 1000, K1)
    bonus = 4242
    for pattern in range(1 << K1):
        match = [(pattern >> j) & 1 for j in range(K1)]
        target = [int(draft[j]) if match[j] else int(draft[j]) + 1
                  for j in range(K1)] + [bonus]
        lead = 0
        for m in match:
            if not m:
                break
            lead += 1
        acc, nxt = verify_greedy(draft, target)
        assert acc == lead + 1
        assert nxt == target[lead]


def _exhaustive_expectation(p):
    k1 = len(p)
    total = 0.0
    for bits in itertools.product([0, 1], repeat=k1):
        prob = 1.0
        for pj, b in zip(p, bits):
            prob *= pj if b else 1.0 - pj
        lead = 0
        for b in bits:
            if not b:
                break
            lead += 1
        total += prob * (lead + 1)
    return total


@pytest.mark.parametrize("name", ["tiny-f32", "qwen3-8b-3L-b4-ctx32k",
                                  "qwen3-8b-3L-b64-ctx256-2k-S2"])
def test_expected_accept_len_closed_form_vs_enumeration(name):
    p = W.WORKLOADS[name].match_probs()
    assert np.isclose(expected_accept_len(p), _exhaustive_expectation(p),
                      rtol=1e-12)


def test_expected_accept_len_values():
    assert round(expected_accept_len([0.8] * 15), 4) == 4.8593
    assert round(expected_accept_len([0.75] * 15), 4) == 3.9599
    p = W.WORKLOADS["qwen3-8b-3L-b4-ctx32k"].match_probs()
    assert np.isclose(p[0], 0.9) and np.isclose(p[-1], 0.34)
    assert round(expected_accept_len(p), 4) == 4.8232


def test_synthetic_target_statistics_and_mismatch():
    wl = W.WORKLOADS["tiny-f32"].replace(batch=20000)
    d = W.gen_verify_draws(wl)
    rng = np.random.default_rng(1)
    draft = rng.integers(0, wl.vocab, (wl.batch, 15))
    T = synthetic_target(draft, d["u"], d["r"], d["tail"], d["p"], wl.vocab)
    agree = T[:, :15] == draft
    # a disagreement never lands on the draft by accident
    assert ((d["u"] < d["p"]) == agree).all()
    assert T.min() >= 0 and T.max() < wl.vocab
    acc = np.array([verify_greedy(draft[b], T[b])[0]
                    for b in range(wl.batch)])
    mu = expected_accept_len(d["p"])
    sd = acc.std() / np.sqrt(wl.batch)
    assert abs(acc.mean() - mu) < 4 * sd


def _f(prefix):
    """A deterministic 'target model': next greedy token from a hash."""
    h = hashlib.sha256(np.asarray(prefix, dtype=np.int64).tobytes())
    return int.from_bytes(h.digest()[:4], "little") % 50


@pytest.mark.parametrize("drafter", ["random", "oracle-like", "perfect"])
def test_losslessness_draft_verify_loop(drafter):
    # whatever the drafts are, the accepted stream equals the target's own
    # greedy stream (anchor hand-off and bonus indexing included)
    rng = np.random.default_rng(2)
    K, N = 16, 300
    ref = [7]
    while len(ref) < N + K + 2:
        ref.append(_f(ref))
    y = [7]                        # verified tokens (their states exist)
    anchor = _f(y)                 # target token carried into the block
    rounds = 0
    while len(y) < N:
        if drafter == "random":
            d = list(rng.integers(0, 50, K - 1))
        elif drafter == "perfect":
            d, s = [], y + [anchor]
            for _ in range(K - 1):
                d.append(_f(s))
                s = s + [d[-1]]
        else:                      # right for a while, then wrong
            d, s = [], y + [anchor]
            cut = int(rng.integers(0, K))
            for j in range(K - 1):
                t = _f(s)
                d.append(t if j < cut else (t + 1) % 50)
                s = s + [d[-1]]
        block = [anchor] + d
        target = [_f(y + block[:j + 1]) for j in range(K)]
        acc, nxt = verify_greedy(d, target)
        y = y + block[:acc]        # anchor plus tau accepted drafts
        anchor = nxt
        rounds += 1
    assert y[:N] == ref[:N]
    if drafter == "perfect":
        assert rounds <= (N + K - 1) // K + 1


def test_latency_formula_matches_tick_simulation():
    rng = np.random.default_rng(3)
    for _ in range(50):
        gamma = int(rng.integers(1, 17))
        t_step = int(rng.integers(1, 5))
        t_ver = int(rng.integers(1, 30))
        taus = list(rng.integers(0, gamma + 1, 20))
        per, overall = simulate_rounds(gamma, t_step, t_ver, taus)
        for tau, got in zip(taus, per):
            assert got == latency_per_token(gamma * t_step, t_ver, tau)
        assert overall == Fraction(len(taus) * (gamma * t_step + t_ver),
                                   sum(taus) + len(taus))
    # block drafter: S passes instead of gamma steps
    per, _ = simulate_rounds(2, 3, 12, [4])
    assert per[0] == latency_per_token(2 * 3, 12, 4) == Fraction(18, 5)


def test_toy_race_printed_values():
    with open(os.path.join(GOLDEN, "toy_race.json")) as fh:
        gold = json.load(fh)
    for case in gold["cases"]:
        K, S, v = case["K"], case["S"], gold["verify_ticks"]
        ar, blk, acc, ratio = simulate_toy_race(K, S, v, cycles=37)
        assert ratio == toy_race_ratio(K, S, v)
        assert round(float(ratio), case["printed_rounding_digits"]) == float(
            case["printed"])
    assert toy_race_ratio(8, 2) == Fraction(20, 14)
    assert toy_race_ratio(16, 2) == 2
