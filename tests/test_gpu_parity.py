"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Inputs come from the seeded ``workloads`` generators and are handed to both
sides unchanged; nothing the GPU computes is fed to the oracle.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import (OracleModel, draft_batch, inject_rows, synthetic_target,
                    verify_greedy as oracle_verify)
from tests.gpu_common import (DEV, MARGIN_MIN, Float32Floor, anchor_blocks,
                              cache_rows, check_bf16_close, check_pass,
                              check_single_pass, check_two_pass, f64,
                              pass_items, say, to_dev)

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")


def small_s2(**kw):
    return W.small_bf16(num_passes=2, commit_per_pass=8, name="small-bf16-S2",
                        **kw)


# Batch sizes pick the GEMM paths: 3 sequences (48 block rows) stream the
# weights with wide workgroups; 8 (128 rows) and 36 (576 rows) take the
# LDS-tiled MFMA kernel with 64x64 and 128x128 blocks (as do the LM head
# and the injection of every prefix above 64 rows); the LM head of 24 and
# 36 sequences (360 and 540 rows) takes 256x256 blocks on sixteen waves,
# with ragged row and column tails.  One sequence (15 LM-head
# rows) takes the persistent LM head: its vocabulary of 8272 = 517 tiles of
# 16 gives each of 256 workgroups two or three tiles (one each for tiny-f32);
# its hidden size of 4096 gives the projections long contractions with few
# column tiles, as in the Qwen3-8B-shaped drafters.
WLS = {
    "tiny-f32": W.WORKLOADS["tiny-f32"],
    "wide-bf16-b1": W.small_bf16(batch=1, hidden=4096, intermediate=2048,
                                 vocab=8272, ctx_min=200, ctx_max=200,
                                 name="wide-bf16-b1", seed=80),
    "small-bf16": W.small_bf16(),
    "small-bf16-b8": W.small_bf16(batch=8, ctx_min=20, ctx_max=150,
                                  name="small-bf16-b8", seed=78),
    "small-bf16-b36": W.small_bf16(batch=36, ctx_min=16, ctx_max=80,
                                   name="small-bf16-b36", seed=79),
    "small-bf16-b24": W.small_bf16(batch=24, ctx_min=16, ctx_max=120,
                                   name="small-bf16-b24", seed=100),
    # the other two query-group sizes the attention kernel is specialised
    # for: 2 (with head_dim 128, streaming GEMMs) and 8 (tiled GEMMs)
    "small-bf16-g2-d128": W.small_bf16(num_q_heads=4, num_kv_heads=2,
                                       head_dim=128, name="small-bf16-g2-d128",
                                       seed=81),
    "small-bf16-g8-b8": W.small_bf16(num_q_heads=16, num_kv_heads=2, batch=8,
                                     ctx_min=30, ctx_max=260,
                                     name="small-bf16-g8-b8", seed=82),
    # a 256-wide drafter at batch 1: the persistent LM head and the chunked
    # projection streams with fewer contraction steps than waves
    "small-bf16-h256-b1": W.small_bf16(batch=1, hidden=256, num_q_heads=4,
                                       num_kv_heads=2, head_dim=64,
                                       intermediate=704, ctx_min=90,
                                       ctx_max=90, name="small-bf16-h256-b1",
                                       seed=99),
    # 16 sequences (256 block rows, 240 LM-head rows): the LM head in one
    # 256-row block on eight waves, and a SwiGLU output of 16512 columns (a
    # multiple of 192) in 128 x 192 blocks
    "small-bf16-b16-ffn": W.small_bf16(batch=16, intermediate=8256,
                                       ctx_min=20, ctx_max=120,
                                       name="small-bf16-b16-ffn", seed=98),
    # 36 sequences (576 block rows) with that SwiGLU output: 128 x 128
    # blocks with a ragged last row block
    "small-bf16-b36-ffn": W.small_bf16(batch=36, intermediate=8256,
                                       ctx_min=16, ctx_max=80,
                                       name="small-bf16-b36-ffn", seed=101),
}


def _setup(wl, random_gains=False, max_ctx=None):
    w_cpu = W.gen_weights(wl, random_gains=random_gains)
    w_dev = to_dev(w_cpu)
    ctx = dfl.DFlash(wl, w_dev, max_ctx=max_ctx)
    return w_cpu, w_dev, ctx


# ------------------------------------------------------------- verify -----

def test_verify_all_patterns_bit_exact():
    K1 = 15
    B = 1 << K1
    rng = np.random.default_rng(0)
    draft = rng.integers(0, 151936, (B, K1)).astype(np.int32)
    pat = np.arange(B)[:, None] >> np.arange(K1)[None, :] & 1
    target = np.concatenate([np.where(pat == 1, draft, draft + 1),
                             rng.integers(0, 151936, (B, 1))], 1).astype(np.int32)
    acc, nxt = dfl.verify_greedy(torch.from_numpy(draft).to(DEV),
                                 torch.from_numpy(target).to(DEV))
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    for b in range(0, B, 7):
        a, n = oracle_verify(draft[b], target[b])
        assert acc[b] == a and nxt[b] == n
    lead = np.argmin(np.concatenate([pat, np.zeros((B, 1), int)], 1), 1)
    np.testing.assert_array_equal(acc, lead + 1)


def test_synthetic_target_harness_matches_oracle():
    wl = W.WORKLOADS["qwen3-8b-3L-b4-ctx32k"].replace(batch=512)
    d = W.gen_verify_draws(wl)
    rng = np.random.default_rng(1)
    draft = rng.integers(0, wl.vocab, (wl.batch, 15)).astype(np.int32)
    T = dfl.synth_target(*(torch.from_numpy(a).to(DEV) for a in (
        draft, d["u"], d["r"], d["tail"], d["p"])), wl.vocab)
    ref = synthetic_target(draft, d["u"], d["r"], d["tail"], d["p"], wl.vocab)
    np.testing.assert_array_equal(T.cpu().numpy(), ref)


# ------------------------------------------------------------ inject ------

@pytest.mark.parametrize("name", list(WLS))
@pytest.mark.parametrize("gains", [False, True])
def test_inject_kv_parity(name, gains):
    wl = WLS[name]
    say(f"[inject] {name} random_gains={gains}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=gains)
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
    kv = ctx.new_kv_cache()
    # two calls with ragged row counts, rows of several sequences interleaved
    seqs, poss = [], []
    for b, L in enumerate(lens):
        seqs += [b] * int(L)
        poss += list(range(int(L)))
    seqs, poss = np.array(seqs), np.array(poss)
    perm = np.random.default_rng(2).permutation(len(seqs))
    seqs, poss = seqs[perm], poss[perm]
    H = W.gen_hiddens(wl, len(seqs))
    cut = len(seqs) // 3 + 1
    for lo, hi in ((0, cut), (cut, len(seqs))):
        ctx.inject_kv([h[lo:hi].to(DEV) for h in H],
                      torch.from_numpy(seqs[lo:hi].astype(np.int32)).to(DEV),
                      torch.from_numpy(poss[lo:hi].astype(np.int32)).to(DEV),
                      kv)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    ref = inject_rows(model, H, poss)
    for l in range(wl.num_layers):
        for b, L in enumerate(lens):
            sel = np.nonzero(seqs == b)[0]
            order = np.argsort(poss[sel])
            rk = ref[l][0][sel][order]
            rv = ref[l][1][sel][order]
            gk, gv = cache_rows(kv, l, b, int(L))
            if wl.dtype == "bf16":
                check_bf16_close(gk, rk, f"K l{l} b{b}")
                check_bf16_close(gv, rv, f"V l{l} b{b}")
            else:
                np.testing.assert_allclose(gk, rk, rtol=1e-4, atol=2e-5)
                np.testing.assert_allclose(gv, rv, rtol=1e-4, atol=2e-5)


def test_inject_device_errors_are_reported():
    wl = WLS["small-bf16"]
    _, _, ctx = _setup(wl)
    kv = ctx.new_kv_cache()
    H = [h.to(DEV) for h in W.gen_hiddens(wl, 3)]
    seq = torch.tensor([0, 99, 1], dtype=torch.int32, device=DEV)
    pos = torch.tensor([0, 1, 5], dtype=torch.int32, device=DEV)
    ctx.inject_kv(H, seq, pos, kv)
    bits = ctx.check_device_errors()
    assert bits & 0x4
    pos = torch.tensor([0, 1, 10 ** 6], dtype=torch.int32, device=DEV)
    seq = torch.tensor([0, 1, 1], dtype=torch.int32, device=DEV)
    ctx.inject_kv(H, seq, pos, kv)
    assert ctx.check_device_errors() & 0x8
    assert ctx.check_device_errors() == 0


# ------------------------------------------------------------- draft ------

def _seeded_cache(wl, ctx, lens):
    """Context KV written directly from the seeded generator (shared data)."""
    kv = ctx.new_kv_cache()
    per_seq = []
    for b, L in enumerate(lens):
        d = {}
        for l in range(wl.num_layers):
            k = W.gen_kv_prefix(wl, l, "k", b, int(L), device=DEV)
            v = W.gen_kv_prefix(wl, l, "v", b, int(L), device=DEV)
            kv[l, 0, b, :, :L] = k
            kv[l, 1, b, :, :L] = v
            d[l] = (f64(k).transpose(1, 0, 2), f64(v).transpose(1, 0, 2))
        per_seq.append(d)
    return kv, per_seq


def _gpu_draft(ctx, wl, lens, kv, anchors=None, block=None, S=1, c=0,
               max_len=None):
    B = len(lens)
    K1 = wl.block_size - 1
    draft = torch.full((B, K1), -7, dtype=torch.int32, device=DEV)
    conf = torch.full((B, K1), float("nan"), device=DEV)
    margin = torch.full((B, K1), float("nan"), device=DEV)
    logits = torch.full((S, B, K1, wl.vocab), float("nan"), device=DEV)
    ctx.draft_block(
        torch.from_numpy(np.asarray(lens, np.int32)).to(DEV), kv,
        int(max(lens)) if max_len is None else int(max_len),
        anchor=None if anchors is None else torch.from_numpy(
            np.asarray(anchors, np.int32)).to(DEV),
        block_tokens=None if block is None else torch.from_numpy(
            np.asarray(block, np.int32)).to(DEV),
        num_passes=S, commit_per_pass=c, draft=draft, conf=conf,
        margin=margin, logits=logits)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    return {"draft": draft.cpu().numpy(), "conf": conf.cpu().numpy(),
            "margin": margin.cpu().numpy(), "logits_all": logits.cpu().numpy()}


@pytest.mark.parametrize("name", list(WLS))
def test_draft_single_pass_parity(name):
    wl = WLS[name]
    say(f"[draft S=1] {name}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=True)
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_single_pass(wl, name, g, ref, fl, anchors)


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_draft_two_pass_parity_and_teacher_forcing(batch):
    wl = small_s2(batch=batch)
    say("[draft S=2] small-bf16")
    w_cpu, w_dev, ctx = _setup(wl)
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors, S=2, c=8)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, num_passes=2,
                      commit_per_pass=8, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    teacher = check_two_pass(
        wl, "small-bf16-S2",
        lambda blk: _gpu_draft(ctx, wl, lens, kv, block=blk, S=1), g, ref,
        fl, anchors, c=8)
    tf = _gpu_draft(ctx, wl, lens, kv, block=np.stack(teacher), S=1)
    for b, o in enumerate(ref):
        rows2 = o["masked_rows"][1]
        # caller-committed positions come back as given
        for i in range(1, 16):
            if i not in rows2:
                assert tf["draft"][b, i - 1] == teacher[b][i]
    # bidirectional: changing a later committed token moves an earlier row
    blk2 = np.stack(teacher).copy()
    b0 = 0
    later = max(i for i in range(1, 16) if blk2[b0][i] != wl.mask_id)
    early = min(o for o in ref[b0]["masked_rows"][1])
    if early < later:
        blk2[b0][later] = (blk2[b0][later] + 1) % (wl.vocab - 1)
        tf2 = _gpu_draft(ctx, wl, lens, kv, block=blk2, S=1)
        d = np.abs(tf2["logits_all"][0][b0][early - 1] -
                   tf["logits_all"][0][b0][early - 1]).max()
        assert d > 1e-3


def test_draft_edge_context_lengths():
    """Empty context (block attends only to itself), a single context key,
    the full context capacity (block positions up to max_ctx + 15) and a
    ragged one, in one batch."""
    wl = W.small_bf16(batch=4, name="small-bf16-edge")
    lens = np.array([0, 1, wl.ctx_max, 17], dtype=np.int32)
    say(f"[draft edge] lens {lens.tolist()}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=True)
    model = OracleModel(wl, w_cpu)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_single_pass(wl, wl.name, g, ref, fl, anchors)


def test_draft_single_chunk_attention():
    """Contexts of at most 112 keys: with the 16 block keys every sequence
    fits one attention chunk, so the partial kernel normalises and writes the
    output itself and no merge runs.  Checked against the oracle, and
    bit for bit against the merge path (a larger length bound gives several
    chunks, of which each of these sequences fills only the first)."""
    wl = W.small_bf16(batch=4, name="small-bf16-1chunk")
    lens = np.array([0, 5, 64, 112], dtype=np.int32)
    say(f"[draft one chunk] lens {lens.tolist()}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=True)
    model = OracleModel(wl, w_cpu)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_single_pass(wl, wl.name, g, ref, fl, anchors)
    merged = _gpu_draft(ctx, wl, lens, kv, anchors=anchors,
                        max_len=wl.ctx_max)
    for k in ("draft", "conf", "margin", "logits_all"):
        np.testing.assert_array_equal(g[k], merged[k])


def test_draft_one_chunk_sequences_ordered_by_length():
    """One attention chunk per sequence: the bf16 kernel takes the sequences
    longest first (ranked on the device, equal lengths by index).  Ties,
    empty contexts and several equal maxima must still give every sequence
    its own output rows."""
    wl = W.small_bf16(batch=7, name="small-bf16-ties")
    lens = np.array([64, 30, 64, 0, 30, 64, 7], dtype=np.int32)
    say(f"[draft ties] lens {lens.tolist()}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=True)
    model = OracleModel(wl, w_cpu)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_single_pass(wl, wl.name, g, ref, fl, anchors)


def _deep_chunk(B, Hkv, max_keys, num_cu):
    """The attention plan's chunk for long contexts with few (sequence, kv
    head) pairs: one workgroup per CU, chunks a multiple of 64 keys."""
    target = max(1, -(-num_cu // (B * Hkv)))
    ch = -(-max_keys // target)
    return max(128, -(-ch // 64) * 64)


def test_draft_deep_ring_short_chunks():
    """A length bound of over half a million positions with one sequence
    pair per kv head puts the bf16 attention on its deeper staging ring (one
    workgroup per CU, chunks of thousands of keys).  The contexts end one,
    two and three 64-key tiles into a chunk, so the ring's prologue meets
    chunks shorter than its depth, and one context fills a single chunk."""
    wl = W.small_bf16(batch=4, num_layers=1, name="small-bf16-deep")
    K = wl.block_size
    max_len = 540000
    num_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ch = _deep_chunk(wl.batch, wl.num_kv_heads, max_len + K, num_cu)
    assert ch >= 2048, ch
    lens = np.array([ch + 10 - K, ch + 100 - K, ch + 192 - K, ch - 300],
                    dtype=np.int32)
    say(f"[draft deep ring] chunk {ch}, lens {lens.tolist()}")
    w_cpu, w_dev, ctx = _setup(wl, random_gains=True, max_ctx=max_len)
    model = OracleModel(wl, w_cpu)
    kv, per_seq = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors, max_len=max_len)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_single_pass(wl, wl.name, g, ref, fl, anchors)
    ctx.close()
    del kv
    torch.cuda.empty_cache()


def test_draft_is_deterministic():
    wl = WLS["small-bf16"]
    w_cpu, w_dev, ctx = _setup(wl)
    lens = W.gen_ctx_lens(wl)
    kv, _ = _seeded_cache(wl, ctx, lens)
    anchors = W.gen_anchors(wl)
    a = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    b = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_draft_rows_without_finite_logits_are_flagged():
    """Regression: an LM head whose logits are all NaN leaves a row with no
    argmax (id -1).  The commit flags it (token error bit) and the next
    refinement pass, which embeds every committed id, clamps it into the
    vocabulary instead of reading outside the embedding."""
    wl = WLS["small-bf16"]
    w_cpu, w_dev, _ = _setup(wl)
    w_dev = dict(w_dev)
    w_dev["lm_head"] = torch.full_like(w_dev["lm_head"], float("nan"))
    ctx = dfl.DFlash(wl, w_dev)
    lens = W.gen_ctx_lens(wl)
    kv, _ = _seeded_cache(wl, ctx, lens)
    B, K1 = len(lens), wl.block_size - 1
    draft = torch.full((B, K1), -7, dtype=torch.int32, device=DEV)
    ctx.draft_block(torch.from_numpy(np.asarray(lens, np.int32)).to(DEV), kv,
                    int(max(lens)),
                    anchor=torch.from_numpy(W.gen_anchors(wl)).to(DEV),
                    num_passes=2, commit_per_pass=8, draft=draft)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() & 0x1
    assert (draft.cpu().numpy() == -1).all()
    assert ctx.check_device_errors() == 0


# -------------------------------------------------------- whole step ------

@pytest.mark.parametrize("name", list(WLS))
def test_full_step_inject_draft_verify(name):
    """Inject the whole context, draft, synthetic target, verify."""
    wl = WLS[name]
    say(f"[step] {name}")
    w_cpu, w_dev, ctx = _setup(wl)
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
    kv = ctx.new_kv_cache()
    per_seq, hid_pos = [], []
    for b, L in enumerate(lens):
        H = W.gen_hiddens(wl, int(L), index=b)
        pos = np.arange(int(L), dtype=np.int32)
        ctx.inject_kv([h.to(DEV) for h in H],
                      torch.full((int(L),), b, dtype=torch.int32, device=DEV),
                      torch.from_numpy(pos).to(DEV), kv)
        per_seq.append(inject_rows(model, H, pos))
        hid_pos.append((H, pos))
    anchors = W.gen_anchors(wl)
    g = _gpu_draft(ctx, wl, lens, kv, anchors=anchors)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    # the float32 evaluations inject the whole context themselves
    empty = {l: (np.zeros((0, wl.num_kv_heads, wl.head_dim)),) * 2
             for l in range(wl.num_layers)}
    fl = Float32Floor(wl, w_cpu, [empty] * len(lens), lens,
                      inject=[hp for hp in hid_pos])
    check_single_pass(wl, name, g, ref, fl, anchors)
    d = W.gen_verify_draws(wl)
    dd = {k: torch.from_numpy(v).to(DEV) for k, v in d.items()}
    gdraft = torch.from_numpy(g["draft"]).to(DEV)
    T = dfl.synth_target(gdraft, dd["u"], dd["r"], dd["tail"], dd["p"],
                         wl.vocab)
    acc, nxt = dfl.verify_greedy(gdraft, T)
    acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
    odraft = np.stack([o["draft"] for o in ref])
    oT = synthetic_target(odraft, d["u"], d["r"], d["tail"], d["p"], wl.vocab)
    checked = 0
    for b, o in enumerate(ref):
        a_ref, n_ref = oracle_verify(odraft[b], oT[b])
        # tau is decided by drafted positions 1 .. min(a_ref, K-1): where
        # the GPU drafted the oracle's ids there (every id of margin above
        # 1e-2 unless float32 evaluations flip it too) the verdict is equal
        decisive = range(1, min(a_ref, 15) + 1)
        if all(g["draft"][b, i - 1] == o["tokens"][i] for i in decisive):
            assert acc[b] == a_ref and nxt[b] == n_ref
            checked += 1
        # and the GPU's own verify is exact on its own draft
        assert (acc[b], nxt[b]) == oracle_verify(
            g["draft"][b], T.cpu().numpy()[b])
    say(f"  accept lengths equal to the oracle's end to end: {checked} of "
        f"{len(ref)}")
