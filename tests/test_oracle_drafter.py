"""Pins for the oracle drafter: fusion, injection, attention, the layer, the
LM-head reduction, commit, and the single-pass / bidirectional structure.
CPU only."""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import workloads as W
from oracle import (OracleModel, block_attention, confidence_commit,
                    decoder_layer, draft_batch, fuse_features, inject_kv,
                    inject_rows, lm_head_reduce, round_bf16)
from oracle.drafter import lm_logits


def tiny_f32(**kw):
    base = dict(name="t", num_layers=2, hidden=64, num_q_heads=4,
                num_kv_heads=2, head_dim=16, intermediate=96, vocab=300,
                num_target_layers=3, target_hidden=32, dtype="f32", batch=2,
                ctx_min=5, ctx_max=20, seed=11)
    base.update(kw)
    return W.Workload(**base)


def _rope_complex(x, pos, theta):
    d = x.shape[-1]
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    inv = theta ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * np.asarray(pos)[:, None, None] * inv)
    return np.concatenate([zr.real, zr.imag], axis=-1)


# --------------------------------------------------------------- attention --

def _sdpa_ref(q, keys, vals):
    # torch library attention, non-causal, GQA by repeating kv heads
    group = q.shape[1] // keys.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)              # [Hq, K, d]
    kt = torch.from_numpy(keys).repeat_interleave(group, 1).permute(1, 0, 2)
    vt = torch.from_numpy(vals).repeat_interleave(group, 1).permute(1, 0, 2)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=False)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("L", [0, 1, 37])
def test_block_attention_matches_sdpa(L):
    rng = np.random.default_rng(L)
    q = rng.standard_normal((16, 8, 32))
    keys = rng.standard_normal((L + 16, 2, 32)) * 2.0
    vals = rng.standard_normal((L + 16, 2, 32))
    np.testing.assert_allclose(block_attention(q, keys, vals),
                               _sdpa_ref(q, keys, vals), rtol=1e-12,
                               atol=1e-12)


def test_block_attention_degenerate_cases():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 2, 8))
    # identical keys -> plain mean of the values
    keys = np.repeat(rng.standard_normal((1, 1, 8)), 6, axis=0)
    vals = rng.standard_normal((6, 1, 8))
    o = block_attention(q, keys, vals)
    np.testing.assert_allclose(o, np.broadcast_to(vals.mean(0), o.shape),
                               rtol=1e-13, atol=1e-13)
    # a single key -> its value
    o = block_attention(q, keys[:1], vals[:1])
    np.testing.assert_allclose(o, np.broadcast_to(vals[0], o.shape),
                               rtol=1e-14, atol=1e-14)


# ------------------------------------------------------- fusion/injection --

def test_fusion_matches_torch_linear_and_rms_norm():
    wl = tiny_f32()
    w = W.gen_weights(wl, random_gains=True)
    H = [h.double() for h in W.gen_hiddens(wl, 9)]
    c = fuse_features([h.numpy() for h in H], w["fc"].double().numpy(),
                      w["hidden_norm"].double().numpy(), wl.rms_eps,
                      lambda a: a)
    ref = F.rms_norm(F.linear(torch.cat(H, 1), w["fc"].double()),
                     (wl.hidden,), weight=w["hidden_norm"].double(),
                     eps=wl.rms_eps)
    np.testing.assert_allclose(c, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_injection_brute_force_loops():
    # explicit scalar loops over a tiny drafter vs the vectorised oracle
    wl = tiny_f32(hidden=8, num_q_heads=2, num_kv_heads=2, head_dim=4,
                  target_hidden=4, num_target_layers=2, num_layers=1)
    w = W.gen_weights(wl, random_gains=True)
    H = [h.double().numpy() for h in W.gen_hiddens(wl, 3)]
    pos = np.array([0, 5, 40000])
    model = OracleModel(wl, w)
    got = inject_rows(model, H, pos)[0]
    Wfc = w["fc"].double().numpy()
    g = w["hidden_norm"].double().numpy()
    Wk = w["wk"][0].double().numpy()
    Wv = w["wv"][0].double().numpy()
    d, half = 4, 2
    for t in range(3):
        f = []
        for k in range(2):
            for j in range(4):
                f.append(H[k][t, j])
        u = [sum(Wfc[o, i] * f[i] for i in range(8)) for o in range(8)]
        ms = sum(x * x for x in u) / 8.0
        c = [u[o] / math.sqrt(ms + wl.rms_eps) * g[o] for o in range(8)]
        for h in range(2):
            kk = [sum(Wk[h * d + e, i] * c[i] for i in range(8))
                  for e in range(d)]
            vv = [sum(Wv[h * d + e, i] * c[i] for i in range(8))
                  for e in range(d)]
            for i in range(half):
                a = pos[t] * wl.rope_theta ** (-2.0 * i / d)
                k0 = kk[i] * math.cos(a) - kk[i + half] * math.sin(a)
                k1 = kk[i + half] * math.cos(a) + kk[i] * math.sin(a)
                assert abs(got[0][t, h, i] - k0) < 1e-12
                assert abs(got[0][t, h, i + half] - k1) < 1e-12
            for e in range(d):
                assert abs(got[1][t, h, e] - vv[e]) < 1e-12


def test_injection_is_the_layers_own_kv_projection():
    # injected K/V == draft layer l's K/V projection (with RoPE on K) of the
    # fused features, computed here with torch.nn.functional.linear and the
    # complex form of RoPE
    wl = tiny_f32()
    w = W.gen_weights(wl)
    model = OracleModel(wl, w)
    H = [h.double().numpy() for h in W.gen_hiddens(wl, 11)]
    pos = np.arange(100, 111)
    c = fuse_features(H, model.W_fc, model.g_h, wl.rms_eps, model.rnd)
    got = inject_rows(model, H, pos)
    for l in range(wl.num_layers):
        k = F.linear(torch.from_numpy(c), w["wk"][l].double()).numpy()
        v = F.linear(torch.from_numpy(c), w["wv"][l].double()).numpy()
        k = _rope_complex(k.reshape(11, wl.num_kv_heads, wl.head_dim), pos,
                          wl.rope_theta)
        np.testing.assert_allclose(got[l][0], k, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got[l][1], v.reshape(got[l][1].shape),
                                   rtol=1e-12, atol=1e-13)


def test_chunked_injection_equals_one_shot():
    wl = W.small_bf16()
    w = W.gen_weights(wl)
    model = OracleModel(wl, w)
    H = [h for h in W.gen_hiddens(wl, 20)]
    pos = np.arange(20)
    full = inject_rows(model, H, pos)
    a = inject_rows(model, [h[:7] for h in H], pos[:7])
    b = inject_rows(model, [h[7:] for h in H], pos[7:])
    for l in full:
        for i in range(2):
            np.testing.assert_array_equal(
                full[l][i], np.concatenate([a[l][i], b[l][i]]))
            # bf16 drafter stores K/V as bf16 values
            np.testing.assert_array_equal(full[l][i], round_bf16(full[l][i]))


def test_fusion_concat_order():
    # permuting the target layers together with W_fc's column blocks leaves
    # H_cond unchanged; permuting only the layers changes it
    wl = tiny_f32()
    w = W.gen_weights(wl)
    H = [h.double().numpy() for h in W.gen_hiddens(wl, 5)]
    Wfc = w["fc"].double().numpy()
    g = np.ones(wl.hidden)
    Dt = wl.target_hidden
    perm = [2, 0, 1]
    Wp = np.concatenate([Wfc[:, k * Dt:(k + 1) * Dt] for k in perm], axis=1)
    a = fuse_features(H, Wfc, g, 1e-6, lambda x: x)
    b = fuse_features([H[k] for k in perm], Wp, g, 1e-6, lambda x: x)
    c = fuse_features([H[k] for k in perm], Wfc, g, 1e-6, lambda x: x)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    assert np.abs(a - c).max() > 1e-3


# ------------------------------------------------------------ one pass -----

def _torch_pass(wl, w, ctx_k, ctx_v, tokens, L):
    """One drafter pass composed from torch library ops (f32 drafter: no
    storage rounding), logits for every block row."""
    d, Hq, Hkv = wl.head_dim, wl.num_q_heads, wl.num_kv_heads
    K = len(tokens)
    pos = np.arange(L, L + K)
    x = w["embed"].double()[torch.as_tensor(tokens)]
    for l in range(wl.num_layers):
        g = lambda n: w[n][l].double()
        h = F.rms_norm(x, (wl.hidden,), weight=g("attn_norm"), eps=wl.rms_eps)
        q = F.linear(h, g("wq")).numpy().reshape(K, Hq, d)
        k = F.linear(h, g("wk")).numpy().reshape(K, Hkv, d)
        v = F.linear(h, g("wv")).numpy().reshape(K, Hkv, d)
        q, k = _rope_complex(q, pos, wl.rope_theta), _rope_complex(
            k, pos, wl.rope_theta)
        o = _sdpa_ref(q, np.concatenate([ctx_k[l], k]),
                      np.concatenate([ctx_v[l], v]))
        x = x + F.linear(torch.from_numpy(o.reshape(K, Hq * d)), g("wo"))
        h2 = F.rms_norm(x, (wl.hidden,), weight=g("mlp_norm"), eps=wl.rms_eps)
        x = x + F.linear(F.silu(F.linear(h2, g("w_gate"))) *
                         F.linear(h2, g("w_up")), g("w_down"))
    hf = F.rms_norm(x, (wl.hidden,), weight=w["final_norm"].double(),
                    eps=wl.rms_eps)
    return F.linear(hf, w["lm_head"].double()).numpy()


def _random_ctx(wl, L, rng):
    ks = [rng.standard_normal((L, wl.num_kv_heads, wl.head_dim))
          for _ in range(wl.num_layers)]
    vs = [rng.standard_normal((L, wl.num_kv_heads, wl.head_dim))
          for _ in range(wl.num_layers)]
    return ks, vs


def test_single_pass_matches_torch_composition():
    wl = tiny_f32()
    w = W.gen_weights(wl, random_gains=True)
    model = OracleModel(wl, w)
    rng = np.random.default_rng(6)
    L = 13
    ks, vs = _random_ctx(wl, L, rng)
    ctx = {l: (ks[l], vs[l]) for l in range(wl.num_layers)}
    res = draft_batch(model, [ctx], [L], anchors=[42], keep_logits=True)[0]
    tokens = [42] + [wl.mask_id] * 15
    ref = _torch_pass(wl, w, ks, vs, tokens, L)
    np.testing.assert_allclose(res["logits"][0], ref[1:], rtol=1e-10,
                               atol=1e-11)
    np.testing.assert_array_equal(res["draft"], ref[1:].argmax(1))


def test_whole_block_from_one_pass():
    # drafter layers run N_l * S times per block, whatever K is
    for K in (4, 8, 16):
        for S, c in ((1, 0), (2, 2)):
            wl = tiny_f32(block_size=K)
            model = OracleModel(wl, W.gen_weights(wl))
            rng = np.random.default_rng(K)
            ks, vs = _random_ctx(wl, 9, rng)
            ctx = {l: (ks[l], vs[l]) for l in range(wl.num_layers)}
            model.layer_calls = 0
            res = draft_batch(model, [ctx], [9], anchors=[3], num_passes=S,
                              commit_per_pass=c)[0]
            assert model.layer_calls == wl.num_layers * S
            assert len(res["draft"]) == K - 1


def test_block_attention_is_bidirectional_and_reads_context():
    wl = tiny_f32()
    model = OracleModel(wl, W.gen_weights(wl))
    rng = np.random.default_rng(7)
    ks, vs = _random_ctx(wl, 10, rng)
    ctx = {l: (ks[l], vs[l]) for l in range(wl.num_layers)}
    blk = np.full((1, 16), wl.mask_id)
    blk[0, 0], blk[0, 9] = 5, 77           # a committed token at index 9
    base = draft_batch(model, [ctx], [10], block_tokens=blk,
                       keep_logits=True)[0]
    blk2 = blk.copy()
    blk2[0, 9] = 78                        # change only the later token
    alt = draft_batch(model, [ctx], [10], block_tokens=blk2,
                      keep_logits=True)[0]
    # position 1 (before index 9) sees the change: no causal mask
    assert np.abs(base["logits"][0][0] - alt["logits"][0][0]).max() > 1e-6
    # changing one context key changes every drafted position
    ks2 = [k.copy() for k in ks]
    ks2[0][0] += 1.0
    ctx2 = {l: (ks2[l], vs[l]) for l in range(wl.num_layers)}
    alt2 = draft_batch(model, [ctx2], [10], block_tokens=blk,
                       keep_logits=True)[0]
    diff = np.abs(base["logits"][0] - alt2["logits"][0]).max(axis=1)
    assert (diff > 1e-8).all()


def test_shape_contract_two_sequences_prefix_64():
    # the toy harness's shape check (batch 2, prefix 64): one block of drafts
    # per sequence; with an anchor at block index 0 the drafts are K-1 ids
    wl = tiny_f32(batch=2)
    w = W.gen_weights(wl)
    model = OracleModel(wl, w)
    per = []
    for b in range(2):
        H = W.gen_hiddens(wl, 64, index=b)
        per.append(inject_rows(model, H, np.arange(64)))
    out = draft_batch(model, per, [64, 64], anchors=[1, 2])
    draft = np.stack([o["draft"] for o in out])
    assert draft.shape == (2, wl.block_size - 1)
    assert draft.min() >= 0 and draft.max() < wl.vocab


# -------------------------------------------------- LM-head reduction ------

def test_lm_head_reduce_brute_force_with_ties():
    rng = np.random.default_rng(8)
    z = np.round(rng.standard_normal((40, 1024)) * 4, 1)  # many exact ties
    z[3, [10, 500]] = 100.0                               # tie at the top
    red = lm_head_reduce(z)
    for i in range(z.shape[0]):
        row = list(z[i])
        best = max(row)
        assert red["token"][i] == row.index(best)         # lowest id
        srt = sorted(row, reverse=True)
        assert red["top1"][i] == srt[0] and red["top2"][i] == srt[1]
    assert red["margin"][3] == 0.0 and red["token"][3] == 10
    np.testing.assert_allclose(red["lse"], scipy.special.logsumexp(z, axis=1),
                               rtol=1e-14)
    np.testing.assert_allclose(red["conf"],
                               scipy.special.softmax(z, axis=1).max(axis=1),
                               rtol=1e-12)


def test_lm_logits_chunking_matches_one_matmul():
    wl = tiny_f32(vocab=1000)
    w = W.gen_weights(wl)
    model = OracleModel(wl, w)
    x = np.random.default_rng(9).standard_normal((5, wl.hidden))
    a = lm_logits(model, x, chunk=64)
    hf = F.rms_norm(torch.from_numpy(x), (wl.hidden,),
                    weight=w["final_norm"].double(), eps=wl.rms_eps)
    b = F.linear(hf, w["lm_head"].double()).numpy()
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- commit -----

def test_commit_matches_repeated_selection():
    rng = np.random.default_rng(10)
    for trial in range(300):
        K = 16
        conf = np.round(rng.random(K), 1)          # frequent ties
        masked = rng.random(K) < 0.7
        masked[0] = False
        c = int(rng.integers(0, 10))
        got = confidence_commit(conf, masked, c)
        # reference: pick the best remaining position c times
        left = [i for i in range(K) if masked[i]]
        pick = []
        for _ in range(min(c, len(left))):
            best = left[0]
            for i in left:
                if conf[i] > conf[best]:
                    best = i
            pick.append(best)
            left.remove(best)
        assert got == sorted(pick)
    assert confidence_commit(conf, masked, None) == [
        i for i in range(16) if masked[i]]


def test_two_pass_commit_invariants():
    wl = tiny_f32(num_layers=1)
    model = OracleModel(wl, W.gen_weights(wl))
    rng = np.random.default_rng(11)
    ks, vs = _random_ctx(wl, 12, rng)
    ctx = {0: (ks[0], vs[0])}
    res = draft_batch(model, [ctx], [12], anchors=[9], num_passes=2,
                      commit_per_pass=8, keep_logits=True)[0]
    passes = res["pass"][1:]
    assert (passes >= 0).all()                        # nothing left masked
    assert (passes == 0).sum() == 8 and (passes == 1).sum() == 7
    assert len(res["masked_rows"][0]) == 15 and len(res["masked_rows"][1]) == 7
    # positions committed in pass 1 keep their pass-1 token
    for i in np.nonzero(res["pass"] == 0)[0]:
        assert res["tokens"][i] == res["pass_token"][0][i]
    # pass-1 commits are the 8 most confident of the 15
    c1 = res["pass_conf"][0][1:]
    chosen = set(np.nonzero(res["pass"] == 0)[0].tolist())
    worst_in = min(c1[i - 1] for i in chosen)
    best_out = max(c1[i - 1] for i in range(1, 16) if i not in chosen)
    assert worst_in >= best_out
    # the second pass equals a one-pass draft of the committed block
    blk = np.full((1, 16), wl.mask_id)
    blk[0, 0] = 9
    for i in chosen:
        blk[0, i] = res["tokens"][i]
    tf = draft_batch(model, [ctx], [12], block_tokens=blk,
                     keep_logits=True)[0]
    np.testing.assert_array_equal(tf["draft"], res["draft"])
    np.testing.assert_allclose(tf["logits"][0], res["logits"][1], rtol=0,
                               atol=0)
