"""Pins for the speculative-sampling verification in the oracle (CPU).

Each case checks the oracle against something other than its own formula:
the greedy special case (one-hot distributions reduce the rule to the
exact-match prefix), the losslessness theorem (the emitted token is
distributed as the target's p, integrated on a grid of uniforms), hand-worked
inverse-CDF draws, and the acceptance probability min(1, p/q).
"""
import numpy as np
import pytest

from oracle import sample_inverse_cdf, verify_greedy, verify_sampling


def one_hot(ids, V):
    m = np.zeros((len(ids), V), dtype=np.float32)
    m[np.arange(len(ids)), ids] = 1.0
    return m


@pytest.mark.parametrize("seed", range(6))
def test_greedy_special_case_is_the_exact_match_rule(seed):
    rng = np.random.default_rng(seed)
    V, K1 = 9, 15
    for _ in range(40):
        draft = rng.integers(0, V, K1)
        target = np.where(rng.random(K1 + 1) < 0.7,
                          np.concatenate([draft, [0]]), rng.integers(0, V, K1 + 1))
        want = verify_greedy(draft, target)
        q, p = one_hot(draft, V), one_hot(target, V)
        for u in (0.0, 0.3, 0.999):
            got = verify_sampling(draft, q, p, np.full(K1, u, np.float32), u)
            assert got == want


def _emitted_distribution(q, p, p_bonus, N):
    """Distribution of the first emitted token for one drafted position,
    integrated over midpoint grids of the acceptance and sampling uniforms;
    the drafted token x is drawn from q (exact weights)."""
    V = len(q)
    grid = (np.arange(N) + 0.5) / N
    dist = np.zeros(V)
    for x in range(V):
        if q[x] == 0:
            continue
        accepted = np.array([verify_sampling([x], q[None], np.stack([p, p_bonus]),
                                             [u], 0.5)[0] == 2 for u in grid])
        pa = accepted.mean()
        dist[x] += q[x] * pa
        if pa < 1:
            # a uniform that rejects x: the replacement depends on u_sample
            u_rej = grid[np.argmin(accepted)]
            toks = [verify_sampling([x], q[None], np.stack([p, p_bonus]), [u_rej],
                                    us)[1] for us in grid]
            dist += q[x] * (1 - pa) * np.bincount(toks, minlength=V) / N
    return dist


@pytest.mark.parametrize("seed", range(4))
def test_emitted_token_is_distributed_as_the_target(seed):
    rng = np.random.default_rng(100 + seed)
    V, N = 6, 2000
    q = rng.random(V) * (rng.random(V) < 0.8)
    q = (q / q.sum()).astype(np.float32)
    p = rng.random(V) * (rng.random(V) < 0.8)
    p = (p / p.sum()).astype(np.float32)
    dist = _emitted_distribution(q, p, p, N)
    # each acceptance threshold and each cumulative boundary moves a mass of
    # at most 1/N: (1 + V) / N in all
    assert np.abs(dist - p).max() <= (1 + V) / N
    # a rule that resampled from p (not the residual) would be far off
    assert np.abs(q - p).max() > 10 * (1 + V) / N


def test_inverse_cdf_hand_worked():
    w = np.array([0, 0.25, 0, 0.5, 0.25])
    cases = {0.0: 1, 0.24: 1, 0.26: 3, 0.74: 3, 0.76: 4, 0.999: 4}
    for u, want in cases.items():
        assert sample_inverse_cdf(w, u) == want
    # never an index of weight zero, at any u
    for u in np.linspace(0, 0.9999, 997):
        assert w[sample_inverse_cdf(w, u)] > 0


def test_all_accepted_draws_the_bonus_from_the_last_row():
    V, K1 = 5, 3
    q = np.full((K1, V), 0.2, np.float32)
    bonus = np.array([0, 0.25, 0, 0.5, 0.25], np.float32)
    p = np.concatenate([q, bonus[None]])
    for u, want in {0.1: 1, 0.5: 3, 0.9: 4}.items():
        assert verify_sampling([0, 1, 2], q, p, [0.99] * K1, u) == (K1 + 1, want)


def test_acceptance_probability_is_min_one_p_over_q():
    V, N = 4, 1000
    q = np.array([[0.4, 0.2, 0.2, 0.2]], np.float32)
    grid = (np.arange(N) + 0.5) / N
    for px, want in ((0.1, 0.25), (0.4, 1.0), (0.6, 1.0), (0.0, 0.0)):
        rest = (1 - px) / 3
        p = np.array([[px, rest, rest, rest], [0.25] * 4], np.float32)
        acc = np.mean([verify_sampling([0], q, p, [u], 0.5)[0] == 2 for u in grid])
        assert abs(acc - want) <= 1.0 / N


def test_rejection_replacement_avoids_tokens_the_draft_overweights():
    # p(x) < q(x): the residual max(0, p - q) is zero at x, so a rejected x is
    # never the replacement; an id outside the vocabulary is rejected
    q = np.array([[0.7, 0.1, 0.1, 0.1]], np.float32)
    p = np.array([[0.1, 0.3, 0.3, 0.3], [0.25] * 4], np.float32)
    for us in np.linspace(0, 0.999, 50):
        acc, tok = verify_sampling([0], q, p, [0.999], us)
        assert acc == 1 and tok != 0
    acc, tok = verify_sampling([7], q, p, [0.0], 0.5)
    assert acc == 1


def test_identical_distributions_fall_back_to_p():
    # p == q: u * q < p holds for every u < 1, and a forced rejection (u = 1)
    # finds a zero residual and draws from p itself
    q = np.array([[0.5, 0.5, 0.0]], np.float32)
    p = np.array([[0.5, 0.5, 0.0], [0, 0, 1]], np.float32)
    assert verify_sampling([1], q, p, [0.999], 0.9)[0] == 2
    acc, tok = verify_sampling([1], q, p, [1.0], 0.9)
    assert acc == 1 and tok == 1
