"""Paged KV cache at full workload sizes: the benchmark's launch
configuration with the context K/V in shuffled pages of 64 and of 256
positions must give exactly the contiguous cache's results (draft tokens,
confidences, margins and the injected rows), for the 32k-context drafter
(many pages per sequence, many attention chunks and their merge) and the
batch-64 two-pass drafter (one chunk per sequence, the tiled GEMMs'
injection epilogue).  Paging changes only where a position's K/V lives, so
the comparison is bit for bit; the oracle comparison of the same steps is
the full-size parity test.
"""
import gc

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_common import DEV, say

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")

CASES = [("qwen3-8b-3L-b4-ctx32k", 64), ("qwen3-8b-3L-b4-ctx32k", 256),
         ("qwen3-8b-3L-b64-ctx256-2k-S2", 64)]


def _step(ctx, wl, lens, kv, H, row_seq, row_pos):
    B, K1 = wl.batch, wl.block_size - 1
    ctx.inject_kv(H, row_seq, row_pos, kv)
    draft = torch.full((B, K1), -7, dtype=torch.int32, device=DEV)
    conf = torch.full((B, K1), float("nan"), device=DEV)
    margin = torch.full((B, K1), float("nan"), device=DEV)
    ctx.draft_block(torch.from_numpy(lens.astype(np.int32)).to(DEV), kv,
                    int(lens.max()),
                    anchor=torch.from_numpy(W.gen_anchors(wl)).to(DEV),
                    num_passes=wl.num_passes,
                    commit_per_pass=wl.commit_per_pass, draft=draft,
                    conf=conf, margin=margin)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    return draft, conf, margin


@pytest.mark.parametrize("name,ps", CASES)
def test_full_size_paged_matches_contiguous(name, ps):
    wl = W.WORKLOADS[name]
    B, K, n_new = wl.batch, wl.block_size, wl.new_rows
    lens = W.gen_ctx_lens(wl)
    say(f"[paged full size] {name}, pages of {ps}: B={B} "
        f"lens {int(lens.min())}..{int(lens.max())}")
    w_dev = W.gen_weights(wl, device=DEV)
    ctx = dfl.DFlash(wl, w_dev, max_inject_rows=max(2048, B * n_new))
    cfg = ctx.cfg
    kv_c = ctx.new_kv_cache()
    for b, L in enumerate(lens):
        n_pre = int(L) - n_new
        for l in range(wl.num_layers):
            kv_c[l, 0, b, :, :n_pre] = W.gen_kv_prefix(wl, l, "k", b, n_pre,
                                                       device=DEV)
            kv_c[l, 1, b, :, :n_pre] = W.gen_kv_prefix(wl, l, "v", b, n_pre,
                                                       device=DEV)
    H = W.gen_hiddens(wl, B * n_new, device=DEV, index=0, tag="step")
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(np.concatenate(
        [np.arange(int(L) - n_new, int(L)) for L in lens]).astype(
            np.int32)).to(DEV)

    # pages for positions [0, L + K) of every sequence, shuffled; -1 beyond
    need = [(int(L) + K + ps - 1) // ps for L in lens]
    ld = (cfg.max_ctx + K + ps - 1) // ps
    num_pages = sum(need)
    perm = np.random.default_rng(3).permutation(num_pages)
    table = np.full((cfg.max_batch, ld), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[k:k + n]
        k += n
    kv_p = ctx.new_kv_cache_paged(ps, num_pages)
    # the same prefix, moved into the pages one sequence at a time
    for b, L in enumerate(lens):
        n_pre = int(L) - n_new
        pos = torch.arange(n_pre, device=DEV)
        pages = torch.from_numpy(table[b].astype(np.int64)).to(DEV)[pos // ps]
        kv_p[:, :, pages, :, pos % ps, :] = \
            kv_c[:, :, b, :, :n_pre, :].permute(3, 0, 1, 2, 4)

    ref = _step(ctx, wl, lens, kv_c, H, row_seq, row_pos)
    ctx.set_kv_pages(ps, num_pages, torch.from_numpy(table).to(DEV))
    got = _step(ctx, wl, lens, kv_p, H, row_seq, row_pos)
    ctx.set_kv_pages(0)
    for what, g, r in zip(("draft", "conf", "margin"), got, ref):
        assert torch.equal(g, r), f"{what} differs from the contiguous cache"
    # the injected rows and the block's own rows, through the table
    for b, L in enumerate(lens):
        pos = torch.arange(int(L) - n_new, int(L) + K, device=DEV)
        pages = torch.from_numpy(table[b].astype(np.int64)).to(DEV)[pos // ps]
        gathered = kv_p[:, :, pages, :, pos % ps, :]  # [n, Nl, 2, Hkv, d]
        want = kv_c[:, :, b, :, int(L) - n_new:int(L) + K, :].permute(
            3, 0, 1, 2, 4)
        assert torch.equal(gathered, want), f"cache rows differ (seq {b})"
    say(f"  {num_pages} pages: draft, conf, margin and the written rows "
        f"bit-identical")
    del kv_c, kv_p, ctx, w_dev
    gc.collect()
    torch.cuda.empty_cache()
