"""The oracle's bf16 storage points against an independent torch composition
(tests/floor_eval.py), and the float32 floor that the GPU parity bounds of
the deeper drafters rest on.  CPU only.

* In float64 the composition computes the oracle's function with the same
  rounding points, so the two agree to float64 rounding: injected K/V, both
  passes of a two-pass draft, every logit.  Moving one rounding point in the
  oracle (planted in a patched copy, on the CPU) breaks the agreement.
* In float32 (several contraction orders) the composition is a correct
  float32 implementation; how far it lands from the float64 oracle is the
  floor.  At Qwen3-8B shapes that floor grows with the number of draft
  layers (slow test).
"""
import numpy as np
import pytest
import torch

import workloads as W
import oracle.drafter as od
from oracle import OracleModel, draft_batch, inject_rows
from oracle.numerics import rms_norm, rope, silu
from tests import floor_eval


def _small(**kw):
    base = dict(batch=2, ctx_min=30, ctx_max=90, seed=91, name="pin-bf16")
    base.update(kw)
    return W.small_bf16(**base)


def _inputs(wl, L, n_new=16, random_gains=True):
    w = W.gen_weights(wl, random_gains=random_gains)
    prefix = {l: (W.to_f64(W.gen_kv_prefix(wl, l, "k", 0, L - n_new)
                           ).transpose(1, 0, 2),
                  W.to_f64(W.gen_kv_prefix(wl, l, "v", 0, L - n_new)
                           ).transpose(1, 0, 2))
              for l in range(wl.num_layers)}
    H = W.gen_hiddens(wl, n_new, tag="step")
    pos = np.arange(L - n_new, L)
    return w, prefix, H, pos


def _oracle(wl, w, prefix, H, pos, L):
    """Oracle injected K/V and two-pass draft (8 commits in pass 1)."""
    model = OracleModel(wl, w)
    new = inject_rows(model, H, pos)
    ctx = {l: (np.concatenate([prefix[l][0], new[l][0]]),
               np.concatenate([prefix[l][1], new[l][1]]))
           for l in range(wl.num_layers)}
    anchor = int(W.gen_anchors(wl)[0])
    ref = draft_batch(model, [ctx], [L], anchors=[anchor], num_passes=2,
                      commit_per_pass=8, keep_logits=True)[0]
    return new, ref, anchor


def _torch(wl, p, prefix, H, pos, L, ref, anchor, member=0):
    """The composition's K/V, pass-1 logits and pass-2 logits teacher-forced
    with the oracle's pass-1 commits."""
    inj = floor_eval.inject(p, H, pos, member)
    ctx_t = {l: (np.concatenate([prefix[l][0], inj[l][0]]),
                 np.concatenate([prefix[l][1], inj[l][1]]))
             for l in range(wl.num_layers)}
    blk1 = np.full(16, wl.mask_id)
    blk1[0] = anchor
    blk2 = blk1.copy()
    for i in np.nonzero(ref["pass"] == 0)[0]:
        blk2[i] = ref["tokens"][i]
    r1, z1 = floor_eval.pass_logits(p, ctx_t, L, blk1, member)
    r2, z2 = floor_eval.pass_logits(p, ctx_t, L, blk2, member)
    np.testing.assert_array_equal(r1, ref["masked_rows"][0])
    np.testing.assert_array_equal(r2, ref["masked_rows"][1])
    return inj, z1, z2


def _oracle_and_torch(wl, w, prefix, H, pos, L, dtype, member=0):
    new, ref, anchor = _oracle(wl, w, prefix, H, pos, L)
    p = floor_eval.Prepared(wl, w, dtype)
    inj, z1, z2 = _torch(wl, p, prefix, H, pos, L, ref, anchor, member)
    return new, ref, inj, z1, z2


@pytest.mark.parametrize("member", [0, 3])
def test_bf16_rounding_points_match_torch_composition(member):
    wl = _small()
    L = 77
    w, prefix, H, pos = _inputs(wl, L)
    new, ref, inj, z1, z2 = _oracle_and_torch(wl, w, prefix, H, pos, L,
                                              torch.float64, member)
    for l in range(wl.num_layers):
        np.testing.assert_allclose(inj[l][0], new[l][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(inj[l][1], new[l][1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(z1, ref["logits"][0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(z2, ref["logits"][1], rtol=0, atol=1e-12)
    # the oracle's values are bf16 where the drafter stores bf16
    for l in range(wl.num_layers):
        np.testing.assert_array_equal(od.round_bf16(new[l][0]), new[l][0])


def _layer_rounding_variant(which):
    """decoder_layer with one storage point moved (a planted mistake)."""
    def layer(model, l, x, ctx_k, ctx_v, pos):
        P, r = model.L[l], model.rnd
        Kb = x.shape[0]
        model.layer_calls += 1
        h = r(rms_norm(x, P["attn_norm"], model.eps))
        q = r(rope((h @ P["wq"].T).reshape(Kb, model.Hq, model.d), pos,
                   model.theta))
        kraw = (h @ P["wk"].T).reshape(Kb, model.Hkv, model.d)
        if which == "k_before_rope":
            k = rope(r(kraw), pos, model.theta)
        else:
            k = r(rope(kraw, pos, model.theta))
        v = (h @ P["wv"].T).reshape(Kb, model.Hkv, model.d)
        if which != "v_unrounded":
            v = r(v)
        keys = np.concatenate([ctx_k, k], axis=0)
        vals = np.concatenate([ctx_v, v], axis=0)
        o = od.block_attention(q, keys, vals)
        if which != "o_unrounded":
            o = r(o)
        o = o.reshape(Kb, model.Hq * model.d)
        x = x + o @ P["wo"].T
        h2 = r(rms_norm(x, P["mlp_norm"], model.eps))
        a = silu(h2 @ P["w_gate"].T) * (h2 @ P["w_up"].T)
        if which != "act_unrounded":
            a = r(a)
        return x + a @ P["w_down"].T
    return layer


@pytest.mark.parametrize("which", ["k_before_rope", "v_unrounded",
                                   "o_unrounded", "act_unrounded"])
def test_moved_rounding_point_is_detected(which, monkeypatch):
    wl = _small(num_layers=1)
    L = 50
    w, prefix, H, pos = _inputs(wl, L)
    # the unpatched layer reproduces the oracle, so the copy is faithful
    monkeypatch.setattr(od, "decoder_layer", _layer_rounding_variant("none"))
    _, ref, _, z1, _ = _oracle_and_torch(wl, w, prefix, H, pos, L,
                                         torch.float64)
    np.testing.assert_allclose(z1, ref["logits"][0], rtol=0, atol=1e-12)
    monkeypatch.setattr(od, "decoder_layer", _layer_rounding_variant(which))
    _, ref, _, z1, _ = _oracle_and_torch(wl, w, prefix, H, pos, L,
                                         torch.float64)
    assert np.abs(z1 - ref["logits"][0]).max() > 1e-6


def test_float32_evaluation_is_a_float32_distance_away():
    """The float32 composition is close to, but not at, the oracle."""
    wl = _small()
    L = 77
    w, prefix, H, pos = _inputs(wl, L)
    _, ref, _, z1, _ = _oracle_and_torch(wl, w, prefix, H, pos, L,
                                         torch.float32)
    d = np.abs(z1 - ref["logits"][0]).max()
    assert 1e-6 < d < 2e-2


@pytest.mark.slow
def test_float32_floor_grows_with_draft_layers():
    """Qwen3-8B shapes, context 2048, one sequence: the largest logit
    distance of four float32 evaluations from the oracle, for 1, 3 and 5
    draft layers."""
    torch.set_num_threads(8)
    floors = []
    for nl in (1, 3, 5):
        wl = W.WORKLOADS["qwen3-8b-1L-b1-ctx2048"].replace(num_layers=nl)
        L = 2048
        w, prefix, H, pos = _inputs(wl, L, random_gains=False)
        _, ref, anchor = _oracle(wl, w, prefix, H, pos, L)
        p = floor_eval.Prepared(wl, w, torch.float32)
        worst = 0.0
        for m in range(4):
            _, z1, z2 = _torch(wl, p, prefix, H, pos, L, ref, anchor, m)
            worst = max(worst, np.abs(z1 - ref["logits"][0]).max(),
                        np.abs(z2 - ref["logits"][1]).max())
        floors.append(worst)
        print(f"{nl} draft layer(s): float32 floor {worst:.3e}", flush=True)
        del w, prefix, p
    assert 1.2e-2 < floors[0] < 3e-2
    assert floors[0] < floors[1] < floors[2] < 8e-2
