"""A whole drafting step captured once in a HIP graph and replayed.

The step is: inject the 16 new context rows of every sequence, draft the
block (one or two passes), derive the synthetic target's greedy tokens,
verify.  The three drafting calls only enqueue kernels on the given stream
(no allocation, no synchronisation, no host read-back), so a graph holds the
whole step.  Every replay must reproduce the eager step bit for bit; eager
work and synchronisation run between the replays.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, say, to_dev

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")

# 8 sequences take the tiled GEMMs (64x64 blocks, split-K for the residual
# projections); 3 sequences with two passes take the streaming GEMMs and the
# confidence-ordered commit.
CASES = {
    "small-bf16-b8": W.small_bf16(batch=8, ctx_min=20, ctx_max=150,
                                  name="small-bf16-b8", seed=78),
    "small-bf16-S2": W.small_bf16(num_passes=2, commit_per_pass=8,
                                  name="small-bf16-S2"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_replays_in_a_hip_graph(name):
    wl = CASES[name]
    say(f"[graph] {name}")
    B, K, n_new = wl.batch, wl.block_size, wl.new_rows
    ctx = dfl.DFlash(wl, to_dev(W.gen_weights(wl)))
    lens = W.gen_ctx_lens(wl)
    kv = ctx.new_kv_cache()
    # context before the new rows, injected eagerly
    for b, L in enumerate(lens):
        n_pre = int(L) - n_new
        if n_pre <= 0:
            continue
        H = W.gen_hiddens(wl, n_pre, index=b, tag="prefix")
        ctx.inject_kv([h.to(DEV) for h in H],
                      torch.full((n_pre,), b, dtype=torch.int32, device=DEV),
                      torch.arange(n_pre, dtype=torch.int32, device=DEV), kv)
    # the step's inputs and outputs, all allocated before capture
    H = [h.to(DEV) for h in W.gen_hiddens(wl, B * n_new, index=0, tag="step")]
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(np.concatenate(
        [np.arange(int(L) - n_new, int(L)) for L in lens]).astype(
            np.int32)).to(DEV)
    ctx_len = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    anchor = torch.from_numpy(W.gen_anchors(wl)).to(DEV)
    d = {k: torch.from_numpy(v).to(DEV)
         for k, v in W.gen_verify_draws(wl).items()}
    draft = torch.empty(B, K - 1, dtype=torch.int32, device=DEV)
    conf = torch.empty(B, K - 1, dtype=torch.float32, device=DEV)
    target = torch.empty(B, K, dtype=torch.int32, device=DEV)
    accept = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    outs = (draft, conf, target, accept, nxt)
    max_len = int(lens.max())

    def step():
        ctx.inject_kv(H, row_seq, row_pos, kv)
        ctx.draft_block(ctx_len, kv, max_len, anchor=anchor,
                        num_passes=wl.num_passes,
                        commit_per_pass=wl.commit_per_pass, draft=draft,
                        conf=conf)
        dfl.synth_target(draft, d["u"], d["r"], d["tail"], d["p"], wl.vocab,
                         target=target)
        dfl.verify_greedy(draft, target, accept=accept, next_anchor=nxt)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert ctx.check_device_errors() == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:  # eager work between the replays
            t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), f"replay {rep} differs from eager"
        say(f"  replay {rep}: draft, confidence, target, accept equal eager")
    assert ctx.check_device_errors() == 0


def test_graph_captured_at_capacity_follows_growing_contexts():
    """A serving loop replays one captured step while every context grows.
    The attention grid is sized at capture from the host's length bound, so
    the step is captured with the bound at the cache capacity (max_ctx);
    before each replay the step's new hidden states, their positions and
    the context lengths are rewritten in place (16 more rows per sequence
    each time).  Every replay equals the same step run eagerly with the same
    bound on a second cache, bit for bit, and agrees with the oracle."""
    from oracle import OracleModel, draft_batch, inject_rows
    from tests.gpu_common import Float32Floor, check_single_pass

    wl = W.small_bf16(batch=3, ctx_min=40, ctx_max=120, name="small-bf16-grow",
                      seed=83)
    B, K, n_new, reps = wl.batch, wl.block_size, wl.new_rows, 3
    say("[graph, growing contexts] small-bf16, 3 sequences")
    w_cpu = W.gen_weights(wl)
    max_ctx = 256
    ctx = dfl.DFlash(wl, to_dev(w_cpu), max_ctx=max_ctx)
    lens0 = W.gen_ctx_lens(wl)
    kv, kv_e = ctx.new_kv_cache(), ctx.new_kv_cache()
    prefix_h = []
    for b, L in enumerate(lens0):  # context before the first step's rows
        n_pre = int(L) - n_new
        H = W.gen_hiddens(wl, n_pre, index=b, tag="prefix")
        prefix_h.append(H)
        for cache in (kv, kv_e):
            ctx.inject_kv([h.to(DEV) for h in H],
                          torch.full((n_pre,), b, dtype=torch.int32,
                                     device=DEV),
                          torch.arange(n_pre, dtype=torch.int32, device=DEV),
                          cache)
    step_h = [W.gen_hiddens(wl, B * n_new, index=r, tag="step")
              for r in range(reps)]

    def positions(r):
        lens = lens0 + n_new * r
        pos = np.concatenate([np.arange(int(L) - n_new, int(L))
                              for L in lens]).astype(np.int32)
        return lens, pos

    H = [h.to(DEV) for h in step_h[0]]
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(positions(0)[1]).to(DEV)
    ctx_len = torch.from_numpy(lens0.astype(np.int32)).to(DEV)
    anchor = torch.from_numpy(W.gen_anchors(wl)).to(DEV)
    draft = torch.empty(B, K - 1, dtype=torch.int32, device=DEV)
    conf = torch.empty(B, K - 1, dtype=torch.float32, device=DEV)
    margin = torch.empty(B, K - 1, dtype=torch.float32, device=DEV)
    logits = torch.empty(1, B, K - 1, wl.vocab, device=DEV)
    outs = (draft, conf, margin, logits)

    def step(cache):
        ctx.inject_kv(H, row_seq, row_pos, cache)
        ctx.draft_block(ctx_len, cache, max_ctx, anchor=anchor, draft=draft,
                        conf=conf, margin=margin, logits=logits)

    # capture on a scratch copy of the cache (capture runs nothing)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(kv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(kv)
    torch.cuda.synchronize()

    model = OracleModel(wl, w_cpu)
    anchors = W.gen_anchors(wl)
    for r in range(reps):
        lens, pos = positions(r)
        for h, src in zip(H, step_h[r]):
            h.copy_(src.to(DEV))
        row_pos.copy_(torch.from_numpy(pos))
        ctx_len.copy_(torch.from_numpy(lens.astype(np.int32)))
        step(kv_e)  # eager, same bound, second cache
        torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        for t in outs:
            t.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip(outs, want):
            assert torch.equal(t, w), f"replay {r} differs from eager"
        assert ctx.check_device_errors() == 0
        # the oracle, from every row injected so far
        per_seq, hid_pos = [], []
        for b, L in enumerate(lens):
            rows = [torch.cat([prefix_h[b][k]] +
                              [step_h[q][k][b * n_new:(b + 1) * n_new]
                               for q in range(r + 1)])
                    for k in range(wl.num_target_layers)]
            p_b = np.arange(int(L))
            per_seq.append(inject_rows(model, rows, p_b))
            hid_pos.append((rows, p_b))
        ref = draft_batch(model, per_seq, lens, anchors=anchors,
                          keep_logits=True)
        empty = {l: (np.zeros((0, wl.num_kv_heads, wl.head_dim)),) * 2
                 for l in range(wl.num_layers)}
        fl = Float32Floor(wl, w_cpu, [empty] * B, lens, inject=hid_pos)
        g = {"draft": draft.cpu().numpy(), "conf": conf.cpu().numpy(),
             "margin": margin.cpu().numpy(),
             "logits_all": logits.cpu().numpy().astype(np.float64)}
        check_single_pass(wl, f"replay {r} (contexts {lens.tolist()})", g,
                          ref, fl, anchors)
