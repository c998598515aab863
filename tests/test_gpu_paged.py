"""Paged KV cache: the same drafting step with the context K/V stored in
pages must give bit-identical results to the contiguous cache.

Paging changes only where a position's K/V lives (a block table maps each
sequence's page index to a page of a shared pool), not what is computed, so
the comparison is exact: draft tokens, confidences and margins, and every
cached K/V row gathered back through the table.  Pages are handed out in a
random order, context lengths are ragged and cross page boundaries, and the
table entries past a sequence's last needed page hold -1, so a read of any
of them would raise the page error bit.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import OracleModel, draft_batch, inject_rows
from tests.gpu_common import (DEV, Float32Floor, check_bf16_close,
                              check_single_pass, f64, say, to_dev)

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")

DEVERR_PAGE = 0x10

# (workload, page size): both GEMM families (streaming, tiled), f32 and bf16,
# head_dim 64 and 128, one and two refinement passes
CASES = {
    "tiny-f32-p64": (W.WORKLOADS["tiny-f32"], 64),
    "small-bf16-S2-p128": (W.small_bf16(num_passes=2, commit_per_pass=8,
                                        name="small-bf16-S2"), 128),
    "small-bf16-b8-p64": (W.small_bf16(batch=8, ctx_min=20, ctx_max=150,
                                       name="small-bf16-b8", seed=78), 64),
    "small-bf16-g2-d128-p64": (W.small_bf16(num_q_heads=4, num_kv_heads=2,
                                            head_dim=128,
                                            name="small-bf16-g2-d128",
                                            seed=81), 64),
}


def _step(ctx, wl, kv, lens, outs):
    """Inject every sequence's context, then draft one block."""
    B = wl.batch
    for b, L in enumerate(lens):
        H = W.gen_hiddens(wl, int(L), index=b, tag="prefix")
        ctx.inject_kv([h.to(DEV) for h in H],
                      torch.full((int(L),), b, dtype=torch.int32, device=DEV),
                      torch.arange(int(L), dtype=torch.int32, device=DEV), kv)
    ctx_len = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    anchor = torch.from_numpy(W.gen_anchors(wl)).to(DEV)
    draft, conf, margin = outs
    for t in outs:
        t.fill_(-7)
    ctx.draft_block(ctx_len, kv, int(lens.max()), anchor=anchor,
                    num_passes=wl.num_passes,
                    commit_per_pass=wl.commit_per_pass, draft=draft,
                    conf=conf, margin=margin)
    torch.cuda.synchronize()
    assert B == ctx_len.shape[0]


def _page_table(lens, K, ps, ld, max_batch, seed):
    """Random distinct pages for positions [0, L + K) of each sequence, two
    spare pages that nobody uses, -1 everywhere else."""
    need = [(int(L) + K + ps - 1) // ps for L in lens]
    num_pages = sum(need) + 2
    perm = np.random.default_rng(seed).permutation(num_pages)
    table = np.full((max_batch, ld), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[k:k + n]
        k += n
    return table, num_pages


@pytest.mark.parametrize("name", list(CASES))
def test_paged_cache_matches_contiguous(name):
    wl, ps = CASES[name]
    say(f"[paged] {name}")
    ctx = dfl.DFlash(wl, to_dev(W.gen_weights(wl)))
    K, B = wl.block_size, wl.batch
    cfg = ctx.cfg
    lens = W.gen_ctx_lens(wl)
    mk = lambda: (torch.empty(B, K - 1, dtype=torch.int32, device=DEV),
                  torch.empty(B, K - 1, dtype=torch.float32, device=DEV),
                  torch.empty(B, K - 1, dtype=torch.float32, device=DEV))

    kv_c = ctx.new_kv_cache()
    ref = mk()
    _step(ctx, wl, kv_c, lens, ref)
    assert ctx.check_device_errors() == 0

    ld = (cfg.max_ctx + K + ps - 1) // ps
    table, num_pages = _page_table(lens, K, ps, ld, cfg.max_batch, 5)
    table_d = torch.from_numpy(table).to(DEV)
    kv_p = ctx.new_kv_cache_paged(ps, num_pages)
    assert kv_p.numel() * kv_p.element_size() == \
        dfl.binding.kv_cache_paged_bytes(cfg, ps, num_pages)
    ctx.set_kv_pages(ps, num_pages, table_d)
    got = mk()
    _step(ctx, wl, kv_p, lens, got)
    assert ctx.check_device_errors() == 0, "a page id out of range was read"
    for what, g, r in zip(("draft", "conf", "margin"), got, ref):
        assert torch.equal(g, r), f"{what} differs from the contiguous cache"
    say(f"  {B} sequences, lengths {lens.min()}..{lens.max()}, page {ps}, "
        f"{num_pages} pages: draft, conf, margin bit-identical")

    # every position written (context and the block's own rows) gathered
    # back through the table
    kv_c_h, kv_p_h = kv_c.cpu(), kv_p.cpu()
    for b, L in enumerate(lens):
        pos = np.arange(int(L) + K)
        pages = torch.from_numpy(table[b, pos // ps].astype(np.int64))
        slots = torch.from_numpy(pos % ps)
        # the two index arrays are not adjacent: their dimension comes first
        gathered = kv_p_h[:, :, pages, :, slots, :]  # [n, Nl, 2, Hkv, d]
        want = kv_c_h[:, :, b, :, :int(L) + K, :].permute(3, 0, 1, 2, 4)
        assert torch.equal(gathered, want), f"cache rows differ (seq {b})"
    say("  cached K/V rows identical through the table")

    # a corrupt entry: reads are clamped to page 0 and flagged
    bad = table.copy()
    bad[0, 0] = num_pages
    table_d.copy_(torch.from_numpy(bad))
    ctx.draft_block(torch.from_numpy(lens.astype(np.int32)).to(DEV), kv_p,
                    int(lens.max()),
                    anchor=torch.from_numpy(W.gen_anchors(wl)).to(DEV))
    assert ctx.check_device_errors() & DEVERR_PAGE
    say("  out-of-range page id flagged")

    # back to the contiguous layout
    ctx.set_kv_pages(0)
    again = mk()
    _step(ctx, wl, kv_c, lens, again)
    assert ctx.check_device_errors() == 0
    for g, r in zip(again, ref):
        assert torch.equal(g, r)


def test_set_kv_pages_rejects_bad_geometry():
    wl = W.small_bf16()
    ctx = dfl.DFlash(wl, to_dev(W.gen_weights(wl)))
    cfg = ctx.cfg
    P = cfg.max_ctx + cfg.block_size
    table = torch.zeros(cfg.max_batch, P, dtype=torch.int32, device=DEV)
    for ps in (32, 48, 96, -64):
        with pytest.raises(dfl.DFlashError):
            ctx.set_kv_pages(ps, 4, table)
    with pytest.raises(dfl.DFlashError):  # table_ld * page_size < P
        ctx.set_kv_pages(64, 4, table[:, :(P - 1) // 64].contiguous())
    with pytest.raises(dfl.DFlashError):
        ctx.set_kv_pages(64, 0, table)
    ctx.set_kv_pages(64, 4, table)
    ctx.set_kv_pages(0)
    say("[paged] geometry checks raise")


def test_paged_step_in_a_hip_graph_follows_table_updates():
    """Serving pattern: the step is captured once with a paged cache; the
    block table is device memory read at run time, so moving a sequence's
    pages (copy the page contents, rewrite the table in place) between
    replays must give the same results.  Each replay is also checked
    against the oracle directly: the injected K/V of every sequence
    gathered through the moved table, and the drafted logits, tokens,
    confidences and margins."""
    wl = W.small_bf16(batch=8, ctx_min=20, ctx_max=150, name="small-bf16-b8",
                      seed=78)
    ps = 64
    say("[paged graph] small-bf16-b8, pages of 64")
    w_cpu = W.gen_weights(wl)
    ctx = dfl.DFlash(wl, to_dev(w_cpu))
    K, B, n_new = wl.block_size, wl.batch, wl.new_rows
    cfg = ctx.cfg
    lens = W.gen_ctx_lens(wl)
    ld = (cfg.max_ctx + K + ps - 1) // ps
    table, num_pages = _page_table(lens, K, ps, ld, cfg.max_batch, 11)
    table_d = torch.from_numpy(table).to(DEV)
    kv = ctx.new_kv_cache_paged(ps, num_pages)
    ctx.set_kv_pages(ps, num_pages, table_d)
    for b, L in enumerate(lens):  # context before the step's new rows
        n_pre = int(L) - n_new
        if n_pre <= 0:
            continue
        H = W.gen_hiddens(wl, n_pre, index=b, tag="prefix")
        ctx.inject_kv([h.to(DEV) for h in H],
                      torch.full((n_pre,), b, dtype=torch.int32, device=DEV),
                      torch.arange(n_pre, dtype=torch.int32, device=DEV), kv)
    H = [h.to(DEV) for h in W.gen_hiddens(wl, B * n_new, index=0, tag="step")]
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(np.concatenate(
        [np.arange(int(L) - n_new, int(L)) for L in lens]).astype(
            np.int32)).to(DEV)
    ctx_len = torch.from_numpy(lens.astype(np.int32)).to(DEV)
    anchor = torch.from_numpy(W.gen_anchors(wl)).to(DEV)
    draft = torch.empty(B, K - 1, dtype=torch.int32, device=DEV)
    conf = torch.empty(B, K - 1, dtype=torch.float32, device=DEV)
    margin = torch.empty(B, K - 1, dtype=torch.float32, device=DEV)
    logits = torch.empty(1, B, K - 1, wl.vocab, dtype=torch.float32,
                         device=DEV)

    def step():
        ctx.inject_kv(H, row_seq, row_pos, kv)
        ctx.draft_block(ctx_len, kv, int(lens.max()), anchor=anchor,
                        draft=draft, conf=conf, margin=margin, logits=logits)

    step()
    torch.cuda.synchronize()
    ref = (draft.clone(), conf.clone())
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

    # the oracle: every sequence's context (prefix and the step's rows)
    # injected from the same hidden states, then the draft
    model = OracleModel(wl, w_cpu)
    Hs = W.gen_hiddens(wl, B * n_new, index=0, tag="step")
    per_seq, hid_pos = [], []
    for b, L in enumerate(lens):
        n_pre = max(int(L) - n_new, 0)
        hp = W.gen_hiddens(wl, n_pre, index=b, tag="prefix") if n_pre else None
        rows = [h[b * n_new:(b + 1) * n_new] for h in Hs]
        hb = rows if hp is None else [torch.cat([a, r]) for a, r in
                                      zip(hp, rows)]
        pos = np.concatenate([np.arange(n_pre),
                              np.arange(int(L) - n_new, int(L))])
        per_seq.append(inject_rows(model, hb, pos))
        hid_pos.append((hb, pos))
    anchors = W.gen_anchors(wl)
    ref_or = draft_batch(model, per_seq, lens, anchors=anchors,
                         keep_logits=True)
    empty = {l: (np.zeros((0, wl.num_kv_heads, wl.head_dim)),) * 2
             for l in range(wl.num_layers)}
    fl = Float32Floor(wl, w_cpu, [empty] * B, lens, inject=hid_pos)

    def against_oracle(rep):
        kv_h = kv.cpu()
        for b, L in enumerate(lens):
            pos = np.arange(int(L))
            pages = torch.from_numpy(table[b, pos // ps].astype(np.int64))
            slots = torch.from_numpy(pos % ps)
            got = kv_h[:, :, pages, :, slots, :]  # [L, Nl, 2, Hkv, d]
            for l in range(wl.num_layers):
                check_bf16_close(f64(got[:, l, 0]), per_seq[b][l][0],
                                 f"replay {rep} K l{l} b{b}")
                check_bf16_close(f64(got[:, l, 1]), per_seq[b][l][1],
                                 f"replay {rep} V l{l} b{b}")
        g = {"draft": draft.cpu().numpy(), "conf": conf.cpu().numpy(),
             "margin": margin.cpu().numpy(),
             "logits_all": logits.cpu().numpy().astype(np.float64)}
        check_single_pass(wl, f"paged graph replay {rep}", g, ref_or, fl,
                          anchors)

    rng = np.random.default_rng(12)
    for rep in range(3):
        # move every used page to a new slot of the pool
        used = table[table >= 0]
        new_ids = rng.permutation(num_pages)
        moved = kv.clone()
        moved[:, :, torch.from_numpy(new_ids[used].astype(np.int64)).to(DEV)] = \
            kv[:, :, torch.from_numpy(used.astype(np.int64)).to(DEV)]
        kv.copy_(moved)
        table = np.where(table >= 0, new_ids[np.maximum(table, 0)], -1).astype(
            np.int32)
        table_d.copy_(torch.from_numpy(table))
        draft.fill_(-1)
        conf.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(draft, ref[0]) and torch.equal(conf, ref[1]), \
            f"replay {rep} after moving the pages differs from eager"
        say(f"  replay {rep}: pages moved, draft and confidence equal eager")
        against_oracle(rep)
    assert ctx.check_device_errors() == 0
