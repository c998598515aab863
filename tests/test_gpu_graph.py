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
