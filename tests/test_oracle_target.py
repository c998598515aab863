"""The stand-in target model and the speculative loop around the drafter
(oracle pins, CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import (OracleModel, TargetModel, greedy_stream, round_bf16,
                    speculative_loop, target_forward)


def _tm(wl):
    return TargetModel(W.gen_target_weights(wl))


def test_target_forward_matches_torch_composition():
    wl = W.small_bf16()
    tw = W.gen_target_weights(wl)
    tm = TargetModel(tw)
    toks = [3, 17, 3999 - 1, 0, 1234]
    hooks, nxt, margin = target_forward(tm, toks)
    x = tw["embed"].double()[torch.tensor(toks)]
    for k, (Wk, g) in enumerate(zip(tw["layers"], tw["gains"])):
        u = x + F.linear(x, Wk.double())
        x = torch.from_numpy(round_bf16(F.rms_norm(
            u, (u.shape[-1],), weight=g.double(), eps=tw["eps"]).numpy()))
        np.testing.assert_allclose(hooks[k], x.numpy(), rtol=0, atol=1e-12)
    z = F.linear(x, tw["head"].double()).numpy()
    np.testing.assert_array_equal(nxt, z.argmax(1))
    top = np.sort(z, 1)
    np.testing.assert_allclose(margin, top[:, -1] - top[:, -2], atol=1e-12)


def test_target_rows_are_independent():
    tm = _tm(W.small_bf16())
    toks = list(range(0, 3990, 97))
    h_all, n_all, _ = target_forward(tm, toks)
    for i, t in enumerate(toks):
        h1, n1, _ = target_forward(tm, [t])
        assert n1[0] == n_all[i]
        for k in range(len(h_all)):
            np.testing.assert_array_equal(h1[k][0], h_all[k][i])


def test_greedy_stream_follows_the_head():
    tm = _tm(W.small_bf16())
    s = greedy_stream(tm, 11, 30)
    prev = 11
    for t in s:
        assert t == int(target_forward(tm, [prev])[1][0])
        prev = t


@pytest.mark.parametrize("mode", ["drafter", "right-for-a-while", "perfect"])
def test_loop_emits_the_targets_greedy_stream(mode):
    """Losslessness with target-side capture: whatever the drafts, the
    emitted stream is the target's own greedy stream; the accepted lengths
    follow from the drafts (all 16 when every draft is the target's)."""
    wl = W.small_bf16(batch=1, num_layers=1, seed=95)
    model = OracleModel(wl, W.gen_weights(wl))
    tm = _tm(wl)
    prompt = W.gen_prompt(wl, 24)
    rng = np.random.default_rng(4)
    cuts = {"drafter": None,
            "right-for-a-while": lambda r: int(rng.integers(0, 16)),
            "perfect": lambda r: 15}[mode]
    y, acc = speculative_loop(model, tm, prompt, 60, cuts)
    ref = greedy_stream(tm, int(prompt[-1]), len(y) - len(prompt))
    assert y[:len(prompt)] == [int(t) for t in prompt]
    assert y[len(prompt):] == ref
    assert sum(acc) == len(y) - len(prompt)
    if mode == "perfect":
        assert all(a == 16 for a in acc)
    if mode == "right-for-a-while":
        assert max(acc) > 1
