"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same batch, context capacity and injection capacity, so the
same kernel plans): Qwen3-8B-shaped drafters with 1, 3 and 5 layers, batch 1
to 64, contexts to 32k, one and two passes.

The whole batch runs on the GPU exactly as in a benchmark step (inject the 16
new rows of every sequence, draft, synthetic target, verify); the float64
oracle recomputes a sample of the sequences (the shortest, the longest and
the median context) and the outputs of those sequences are compared element
by element: the injected K/V of all layers, the logits of every drafted row,
the token ids where the oracle's top-2 margin exceeds 1e-2, confidences and
margins.  Verify is compared on every sequence.

The context before the 16 new rows comes from the seeded K/V generator as
data for both sides (injecting 32k rows through the float64 oracle would take
far too long); the new rows are injected by both sides from the same seeded
target hidden states.

Tolerances: the stated bounds (logits max-abs 2e-2, token ids exact where
the top-2 margin exceeds 1e-2), or for the deeper drafters 1.25 times the
largest distance from the oracle of an ensemble of float32 evaluations of
the same inputs, where a token differing at a margin above 1e-2 must be
differed on by one of those evaluations too (tests/gpu_common.py says why).
"""
import gc

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (OracleModel, draft_batch, inject_rows, synthetic_target,
                    verify_greedy as oracle_verify)
from tests.gpu_common import (DEV, Float32Floor, check_bf16_close,
                              check_single_pass, check_two_pass, f64,
                              kv_flip_stats, say)

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")

FULL = [n for n in W.WORKLOAD_ORDER if W.WORKLOADS[n].dtype == "bf16"] + \
    W.EXTRA_WORKLOADS


def sample_seqs(lens):
    order = np.argsort(np.asarray(lens), kind="stable")
    return sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2])})


def gpu_draft(ctx, wl, lens, kv, seqs, anchors=None, block=None, S=1, c=0):
    """Draft the whole batch; return the sampled sequences' outputs."""
    B, K1 = len(lens), wl.block_size - 1
    draft = torch.full((B, K1), -7, dtype=torch.int32, device=DEV)
    conf = torch.full((B, K1), float("nan"), device=DEV)
    margin = torch.full((B, K1), float("nan"), device=DEV)
    logits = torch.full((S, B, K1, wl.vocab), float("nan"), device=DEV)
    ctx.draft_block(
        torch.from_numpy(np.asarray(lens, np.int32)).to(DEV), kv,
        int(max(lens)),
        anchor=None if anchors is None else torch.from_numpy(
            np.asarray(anchors, np.int32)).to(DEV),
        block_tokens=None if block is None else torch.from_numpy(
            np.asarray(block, np.int32)).to(DEV),
        num_passes=S, commit_per_pass=c, draft=draft, conf=conf,
        margin=margin, logits=logits)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    idx = torch.tensor(seqs, device=DEV)
    out = {"draft_all": draft.cpu().numpy(),
           "draft": draft[idx].cpu().numpy(),
           "conf": conf[idx].cpu().numpy().astype(np.float64),
           "margin": margin[idx].cpu().numpy().astype(np.float64),
           "logits_all": logits[:, idx].cpu().numpy().astype(np.float64)}
    del logits
    return out


@pytest.mark.parametrize("name", FULL)
def test_full_size_step_parity(name):
    wl = W.WORKLOADS[name]
    B, n_new, S, c = wl.batch, wl.new_rows, wl.num_passes, wl.commit_per_pass
    lens = W.gen_ctx_lens(wl)
    seqs = sample_seqs(lens)
    say(f"[full size] {name}: B={B} layers={wl.num_layers} S={S} "
        f"lens {int(lens.min())}..{int(lens.max())}, oracle on {seqs}")
    w_dev = W.gen_weights(wl, device=DEV)
    # the benchmark's launch configuration
    ctx = dfl.DFlash(wl, w_dev, max_inject_rows=max(2048, B * n_new))
    kv = ctx.new_kv_cache()
    prefix = {}
    for b, L in enumerate(lens):
        n_pre = int(L) - n_new
        for l in range(wl.num_layers):
            k = W.gen_kv_prefix(wl, l, "k", b, n_pre, device=DEV)
            v = W.gen_kv_prefix(wl, l, "v", b, n_pre, device=DEV)
            kv[l, 0, b, :, :n_pre] = k
            kv[l, 1, b, :, :n_pre] = v
            if b in seqs:
                prefix[(b, l)] = (f64(k).transpose(1, 0, 2),
                                  f64(v).transpose(1, 0, 2))
    H = W.gen_hiddens(wl, B * n_new, device=DEV, index=0, tag="step")
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(np.concatenate(
        [np.arange(int(L) - n_new, int(L)) for L in lens]).astype(
            np.int32)).to(DEV)
    ctx.inject_kv(H, row_seq, row_pos, kv)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    anchors = W.gen_anchors(wl)
    g = gpu_draft(ctx, wl, lens, kv, seqs, anchors=anchors, S=S, c=c)

    # verify of the whole batch against the seeded synthetic target
    d = W.gen_verify_draws(wl)
    T = dfl.synth_target(torch.from_numpy(g["draft_all"]).to(DEV),
                         *(torch.from_numpy(d[k]).to(DEV)
                           for k in ("u", "r", "tail", "p")), wl.vocab)
    acc, nxt = dfl.verify_greedy(torch.from_numpy(g["draft_all"]).to(DEV), T)
    Tn, acc, nxt = T.cpu().numpy(), acc.cpu().numpy(), nxt.cpu().numpy()
    np.testing.assert_array_equal(
        Tn, synthetic_target(g["draft_all"], d["u"], d["r"], d["tail"], d["p"],
                             wl.vocab))
    for b in range(B):
        assert (acc[b], nxt[b]) == oracle_verify(g["draft_all"][b], Tn[b])

    # float64 oracle on the sampled sequences
    w_cpu = {k: ([t.cpu() for t in v] if isinstance(v, list) else v.cpu())
             for k, v in w_dev.items()}
    model = OracleModel(wl, w_cpu)
    Hc = [h.cpu() for h in H]
    per_seq = []
    for b in seqs:
        L = int(lens[b])
        rows = slice(b * n_new, (b + 1) * n_new)
        new = inject_rows(model, [h[rows] for h in Hc], np.arange(L - n_new, L))
        ctx_kv = {}
        for l in range(wl.num_layers):
            gk = f64(kv[l, 0, b, :, L - n_new:L]).transpose(1, 0, 2)
            gv = f64(kv[l, 1, b, :, L - n_new:L]).transpose(1, 0, 2)
            check_bf16_close(gk, new[l][0], f"K l{l} b{b}")
            check_bf16_close(gv, new[l][1], f"V l{l} b{b}")
            ctx_kv[l] = (np.concatenate([prefix[(b, l)][0], new[l][0]]),
                         np.concatenate([prefix[(b, l)][1], new[l][1]]))
        per_seq.append(ctx_kv)
    ref = draft_batch(model, per_seq, lens, anchors=anchors, num_passes=S,
                      commit_per_pass=c, keep_logits=True, seqs=seqs)
    # float32 evaluations of the same step: the same prefix as data, their
    # own injection of the same new rows
    fl = Float32Floor(wl, w_cpu, [{l: prefix[(b, l)] for l in
                                   range(wl.num_layers)} for b in seqs],
                      [lens[b] for b in seqs],
                      inject=[([h[b * n_new:(b + 1) * n_new] for h in Hc],
                               np.arange(int(lens[b]) - n_new, int(lens[b])))
                              for b in seqs])
    for j, b in enumerate(seqs):
        L = int(lens[b])
        for l in range(wl.num_layers):
            gk = f64(kv[l, 0, b, :, L - n_new:L]).transpose(1, 0, 2)
            new_or = per_seq[j][l][0][L - n_new:]
            members = [fl.injected(m, j)[l][0] for m in range(fl.members)]
            kv_flip_stats(gk, new_or, members, f"K l{l} b{b}",
                          quiet=l > 0 or j > 0)
    if S == 1:
        check_single_pass(wl, name, g, ref, fl, [anchors[b] for b in seqs])
    else:
        check_two_pass(wl, name,
                       lambda blk: gpu_draft(ctx, wl, lens, kv, seqs,
                                             block=blk),
                       g, ref, fl, anchors, c, seqs=seqs)
    ctx.close()
    del kv, w_dev, H
    gc.collect()
    torch.cuda.empty_cache()


DEEP = [n for n in FULL if W.WORKLOADS[n].num_layers > 1]


@pytest.mark.parametrize("name", DEEP)
def test_full_size_each_layer_alone(name):
    """Each layer of a deeper drafter run alone as a one-layer drafter (its
    own attention and MLP weights; the shared embedding, fc, final norm and
    LM head; that layer's context K/V) at full size, in the benchmark's
    launch configuration: inject the step's new rows, one pass, against the
    oracle on the sampled sequences.  A defect in any one layer shows here
    at one-layer tolerances, without the other layers' amplification."""
    wl = W.WORKLOADS[name]
    wl1 = wl.replace(num_layers=1, num_passes=1, commit_per_pass=0)
    B, n_new = wl.batch, wl.new_rows
    lens = W.gen_ctx_lens(wl)
    seqs = sample_seqs(lens)
    say(f"[full size, each layer alone] {name}: oracle on {seqs}")
    w_dev = W.gen_weights(wl, device=DEV)
    H = W.gen_hiddens(wl, B * n_new, device=DEV, index=0, tag="step")
    Hc = [h.cpu() for h in H]
    row_seq = torch.arange(B, dtype=torch.int32,
                           device=DEV).repeat_interleave(n_new)
    row_pos = torch.from_numpy(np.concatenate(
        [np.arange(int(L) - n_new, int(L)) for L in lens]).astype(
            np.int32)).to(DEV)
    anchors = W.gen_anchors(wl)
    shared = {k: v.cpu() for k, v in w_dev.items() if not isinstance(v, list)}
    worst = 0.0
    for l in range(wl.num_layers):
        w1 = {k: ([v[l]] if isinstance(v, list) else v)
              for k, v in w_dev.items()}
        ctx = dfl.DFlash(wl1, w1, max_inject_rows=max(2048, B * n_new))
        kv = ctx.new_kv_cache()
        prefix = {}
        for b, L in enumerate(lens):
            n_pre = int(L) - n_new
            k = W.gen_kv_prefix(wl, l, "k", b, n_pre, device=DEV)
            v = W.gen_kv_prefix(wl, l, "v", b, n_pre, device=DEV)
            kv[0, 0, b, :, :n_pre] = k
            kv[0, 1, b, :, :n_pre] = v
            if b in seqs:
                prefix[b] = (f64(k).transpose(1, 0, 2),
                             f64(v).transpose(1, 0, 2))
        ctx.inject_kv(H, row_seq, row_pos, kv)
        g = gpu_draft(ctx, wl1, lens, kv, seqs, anchors=anchors)
        w_cpu = dict(shared)
        for k, v in w_dev.items():
            if isinstance(v, list):
                w_cpu[k] = [v[l].cpu()]
        model = OracleModel(wl1, w_cpu)
        per_seq, inj = [], []
        for b in seqs:
            L = int(lens[b])
            rows = [h[b * n_new:(b + 1) * n_new] for h in Hc]
            pos = np.arange(L - n_new, L)
            new = inject_rows(model, rows, pos)
            per_seq.append({0: (np.concatenate([prefix[b][0], new[0][0]]),
                                np.concatenate([prefix[b][1], new[0][1]]))})
            inj.append((rows, pos))
        ref = draft_batch(model, per_seq, lens, anchors=anchors,
                          keep_logits=True, seqs=seqs)
        fl = Float32Floor(wl1, w_cpu, [{0: prefix[b]} for b in seqs],
                          [lens[b] for b in seqs], inject=inj)
        st = check_single_pass(wl1, f"{name} layer {l} alone", g, ref, fl,
                               [anchors[b] for b in seqs])
        worst = max(worst, st["max_dl"])
        ctx.close()
        del kv, fl, model
        gc.collect()
        torch.cuda.empty_cache()
    say(f"  {name}: worst single layer max |dlogit| {worst:.2e} (stated "
        f"bound 2e-2)")
    del w_dev, H
    gc.collect()
    torch.cuda.empty_cache()
