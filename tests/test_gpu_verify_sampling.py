"""GPU parity of the speculative-sampling verification (temperature > 0)
against the float64 oracle, through the C ABI.

Distributions are seeded softmaxes: the target's p and a draft q that is p
perturbed in logit space (so acceptance varies from position to position),
drafts drawn from q, and uniforms for the acceptance coins and the draw.
Accept lengths must match the oracle exactly (each decision is u * q(x) <
p(x) on float32 inputs, exact in float64 on both sides).  The drawn token
must equal the oracle's, or, where the two sides' float64 running sums are
ordered differently and the target falls within rounding of a boundary, be
a valid draw: of positive weight, with u times the total inside its
cumulative interval up to the rounding of the sums.
"""
import numpy as np
import pytest
import torch

from oracle import verify_greedy as oracle_greedy
from oracle import verify_sampling as oracle_sampling
from tests.gpu_common import DEV, say

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")


def make_case(B, K, V, sigma, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    z = torch.randn(B, K, V, generator=g, device=DEV) * 2.0
    p = torch.softmax(z, -1)
    zq = z[:, :K - 1] + sigma * torch.randn(B, K - 1, V, generator=g, device=DEV)
    q = torch.softmax(zq, -1)
    draft = torch.multinomial(q.reshape(-1, V), 1, generator=g).reshape(B, K - 1)
    ua = torch.rand(B, K - 1, generator=g, device=DEV)
    us = torch.rand(B, generator=g, device=DEV)
    return (draft.to(torch.int32).contiguous(), q.contiguous(), p.contiguous(),
            ua.contiguous(), us.contiguous())


def check_against_oracle(draft, q, p, ua, us, acc, nxt):
    draft, q, p = draft.cpu().numpy(), q.cpu().numpy(), p.cpu().numpy()
    ua, us = ua.cpu().numpy(), us.cpu().numpy()
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    B, K1 = draft.shape
    exact = 0
    for b in range(B):
        a_ref, n_ref = oracle_sampling(draft[b], q[b], p[b], ua[b], us[b])
        assert acc[b] == a_ref, f"seq {b}: accept {acc[b]} vs {a_ref}"
        if nxt[b] == n_ref:
            exact += 1
            continue
        tau = a_ref - 1
        if tau < K1:
            w = np.maximum(p[b, tau].astype(np.float64) - q[b, tau], 0.0)
            if not np.any(w > 0):
                w = p[b, tau].astype(np.float64)
        else:
            w = p[b, K1].astype(np.float64)
        c = np.cumsum(w)
        t = float(np.float32(us[b])) * c[-1]
        x = int(nxt[b])
        tol = 1e-12 * c[-1]
        assert 0 <= x < len(w) and w[x] > 0, f"seq {b}: token {x}"
        lo = c[x - 1] if x > 0 else 0.0
        assert lo - tol <= t <= c[x] + tol, f"seq {b}: {x} vs oracle {n_ref}"
    return exact


@pytest.mark.parametrize("B,V,sigma", [(64, 1000, 0.3), (64, 1000, 1.5),
                                       (16, 151936, 0.5), (3, 63, 0.8)])
def test_verify_sampling_matches_oracle(B, V, sigma):
    K = 16
    draft, q, p, ua, us = make_case(B, K, V, sigma, seed=V + B)
    acc, nxt = dfl.verify_sampling(draft, q, p, ua, us)
    torch.cuda.synchronize()
    exact = check_against_oracle(draft, q, p, ua, us, acc, nxt)
    a = acc.cpu().numpy()
    say(f"[sampling verify] B={B} V={V} sigma={sigma}: accept lengths "
        f"{a.min()}..{a.max()} (mean {a.mean():.2f}), draws equal to the "
        f"oracle's {exact}/{B}")
    # the same inputs give the same outputs
    acc2, nxt2 = dfl.verify_sampling(draft, q, p, ua, us)
    assert torch.equal(acc, acc2) and torch.equal(nxt, nxt2)


def test_one_hot_distributions_reduce_to_greedy():
    B, K, V = 256, 16, 300
    rng = np.random.default_rng(5)
    draft = rng.integers(0, V, (B, K - 1))
    target = np.where(rng.random((B, K)) < 0.8,
                      np.concatenate([draft, np.zeros((B, 1), int)], 1),
                      rng.integers(0, V, (B, K)))
    q = np.zeros((B, K - 1, V), np.float32)
    p = np.zeros((B, K, V), np.float32)
    q[np.arange(B)[:, None], np.arange(K - 1)[None], draft] = 1
    p[np.arange(B)[:, None], np.arange(K)[None], target] = 1
    ua = rng.random((B, K - 1)).astype(np.float32)
    us = rng.random(B).astype(np.float32)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    acc, nxt = dfl.verify_sampling(T(draft.astype(np.int32)), T(q), T(p),
                                   T(ua), T(us))
    gacc, gnxt = dfl.verify_greedy(T(draft.astype(np.int32)),
                                   T(target.astype(np.int32)))
    assert torch.equal(acc, gacc) and torch.equal(nxt, gnxt)
    for b in range(0, B, 17):
        assert (int(acc[b]), int(nxt[b])) == oracle_greedy(draft[b], target[b])


def test_edge_cases():
    K, V = 4, 70  # two tiles, the second ragged
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    rng = np.random.default_rng(9)
    base = rng.random((K, V)).astype(np.float32)
    base /= base.sum(-1, keepdims=True)
    p = base[None].copy()
    q = base[None, :K - 1].copy()
    draft = np.array([[3, 65, 7]], np.int32)
    us = np.array([0.37], np.float32)
    cases = {
        "all accepted (p == q)": (draft, q, p, np.full((1, 3), 0.5, np.float32)),
        "forced rejection, zero residual": (draft, q, p,
                                            np.ones((1, 3), np.float32)),
        "id outside the vocabulary": (np.array([[3, 70, 7]], np.int32), q, p,
                                      np.full((1, 3), 0.5, np.float32)),
        "negative id": (np.array([[-1, 2, 7]], np.int32), q, p,
                        np.full((1, 3), 0.5, np.float32)),
    }
    for name, (d, qq, pp, ua) in cases.items():
        acc, nxt = dfl.verify_sampling(T(d), T(qq), T(pp), T(ua), T(us))
        ref = oracle_sampling(d[0], qq[0], pp[0], ua[0], us[0])
        say(f"  {name}: gpu {(int(acc[0]), int(nxt[0]))} oracle {ref}")
        assert (int(acc[0]), int(nxt[0])) == ref, name
    # a distribution that is zero everywhere draws -1
    pz = p.copy()
    pz[0, K - 1] = 0
    acc, nxt = dfl.verify_sampling(T(draft), T(q), T(pz),
                                   T(np.full((1, 3), 0.5, np.float32)), T(us))
    assert int(acc[0]) == K and int(nxt[0]) == -1
