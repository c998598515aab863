"""dflash_draft_block_noalloc (scratch in the library's static device buffer,
nothing allocated per call) against dflash_draft_block (the context's
workspace): the same kernels on the same inputs, so every output must be
identical bit for bit.  Two calls in a row, the second with a smaller batch,
so the static buffer holds the first call's contents when the second starts.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, say, to_dev

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")


def _inject_prefix(ctx, wl, lens, kv):
    for b, L in enumerate(lens):
        H = [h.to(DEV) for h in W.gen_hiddens(wl, int(L), index=b)]
        ctx.inject_kv(H, torch.full((int(L),), b, dtype=torch.int32,
                                    device=DEV),
                      torch.arange(int(L), dtype=torch.int32, device=DEV), kv)


def _draft(ctx, wl, lens, kv, anchors, noalloc):
    B, K1 = len(lens), wl.block_size - 1
    S, c = wl.num_passes, wl.commit_per_pass
    out = {"draft": torch.full((B, K1), -7, dtype=torch.int32, device=DEV),
           "conf": torch.full((B, K1), float("nan"), device=DEV),
           "margin": torch.full((B, K1), float("nan"), device=DEV),
           "logits": torch.full((S, B, K1, wl.vocab), float("nan"),
                                device=DEV)}
    ctx.draft_block(torch.from_numpy(np.asarray(lens, np.int32)).to(DEV), kv,
                    int(max(lens)),
                    anchor=torch.from_numpy(anchors[:B]).to(DEV),
                    num_passes=S, commit_per_pass=c, draft=out["draft"],
                    conf=out["conf"], margin=out["margin"],
                    logits=out["logits"], noalloc=noalloc)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    return {k: v.cpu().numpy() for k, v in out.items()}


CASES = {
    # streaming GEMMs, persistent LM head, two passes
    "small-bf16-S2": W.small_bf16(num_passes=2, commit_per_pass=8,
                                  name="small-bf16-S2", batch=3),
    # tiled GEMMs with split-K and the tiled LM head
    "small-bf16-b8": W.small_bf16(batch=8, ctx_min=20, ctx_max=150,
                                  name="small-bf16-b8", seed=78),
    "tiny-f32": W.WORKLOADS["tiny-f32"].replace(batch=2, ctx_min=100,
                                                ctx_max=128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_draft_matches_workspace_draft(name):
    wl = CASES[name]
    say(f"[noalloc] {name}: batch {wl.batch}, then 1")
    w_dev = to_dev(W.gen_weights(wl))
    ctx = dfl.DFlash(wl, w_dev)
    kv = ctx.new_kv_cache()
    lens = W.gen_ctx_lens(wl)
    _inject_prefix(ctx, wl, lens, kv)
    torch.cuda.synchronize()
    anchors = W.gen_anchors(wl)
    # batch B, then a smaller batch 1 with a shorter context bound
    for lens_call in (lens, lens[:1]):
        ref = _draft(ctx, wl, lens_call, kv, anchors, noalloc=False)
        got = _draft(ctx, wl, lens_call, kv, anchors, noalloc=True)
        for k in ref:
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        assert (got["draft"] >= 0).all()
    ctx.close()


def test_noalloc_rejects_more_than_the_static_buffer():
    # Qwen3-8B vocabulary with a small trunk: 512 sequences need more than
    # the buffer for their LM-head records alone; nothing is launched
    wl = W.small_bf16(vocab=151936, batch=512, ctx_min=8, ctx_max=8,
                      name="big-vocab", num_layers=1)
    w_dev = to_dev(W.gen_weights(wl))
    ctx = dfl.DFlash(wl, w_dev, max_inject_rows=16)
    kv = ctx.new_kv_cache()
    lens = torch.full((wl.batch,), 8, dtype=torch.int32, device=DEV)
    with pytest.raises(dfl.DFlashError) as e:
        ctx.draft_block(lens, kv, 8,
                        anchor=torch.zeros(wl.batch, dtype=torch.int32,
                                           device=DEV), noalloc=True)
    assert e.value.status == -3 and "static buffer" in str(e.value)
    ctx.close()
