"""Target-side feature capture and the whole speculative loop on the GPU.

The stand-in target model (harness kernel) is checked against its oracle;
then sequences run the pages' loop for many rounds entirely on the GPU: the
target's hooked states of the prompt are injected, each round drafts a block
(dflash_draft_block), the target verifies the block in one pass, greedy
verification keeps the agreed prefix plus the target's own token
(dflash_verify_greedy), and the hooked states of the accepted positions,
computed in that verify pass, are injected before the next block
(dflash_inject_kv).  The emitted stream must be the target's own greedy
stream (losslessness end to end), and it is compared with the oracle's loop.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import (OracleModel, TargetModel, greedy_stream,
                    speculative_loop, target_forward as oracle_target)
from tests.gpu_common import DEV, MARGIN_MIN, check_bf16_close, f64, say, \
    to_dev

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")


def _wl():
    return W.small_bf16(batch=2, num_layers=1, seed=95)


def test_target_kernel_matches_its_oracle_and_is_row_independent():
    wl = _wl()
    tw = W.gen_target_weights(wl)
    twd = {k: ([t.to(DEV) for t in v] if isinstance(v, list) else
               (v.to(DEV) if torch.is_tensor(v) else v))
           for k, v in tw.items()}
    toks = np.random.default_rng(3).integers(0, wl.vocab - 1, 96).astype(
        np.int32)
    hooks, nxt, margin = dfl.target_forward(twd, torch.from_numpy(toks).to(DEV))
    torch.cuda.synchronize()
    h_or, n_or, m_or = oracle_target(TargetModel(tw), toks)
    for k in range(len(hooks)):
        check_bf16_close(f64(hooks[k]), h_or[k], f"hook {k}")
    nx = nxt.cpu().numpy()
    clear = m_or > MARGIN_MIN
    np.testing.assert_array_equal(nx[clear], n_or[clear])
    say(f"[target] next tokens equal the oracle's at {int(clear.sum())} of "
        f"{len(toks)} positions (the rest within {MARGIN_MIN} of a tie)")
    # a position's results do not depend on the others of the launch
    for i in (0, 17, 95):
        h1, n1, m1 = dfl.target_forward(twd, torch.from_numpy(toks[i:i + 1])
                                        .to(DEV))
        assert int(n1[0]) == int(nx[i])
        assert float(m1[0]) == float(margin[i])
        for k in range(len(hooks)):
            assert torch.equal(h1[k][0], hooks[k][i])


@pytest.mark.parametrize("mode", ["drafter", "right-for-a-while"])
def test_speculative_loop_on_gpu_is_lossless(mode):
    wl = _wl()
    B, K, n_emit, L0 = wl.batch, wl.block_size, 64, 24
    say(f"[loop] {mode}: {B} sequences, prompts of {L0}, {n_emit} tokens")
    w_cpu = W.gen_weights(wl)
    tw = W.gen_target_weights(wl)
    twd = {k: ([t.to(DEV) for t in v] if isinstance(v, list) else
               (v.to(DEV) if torch.is_tensor(v) else v))
           for k, v in tw.items()}
    ctx = dfl.DFlash(wl, to_dev(w_cpu), max_ctx=L0 + n_emit + 2 * K)
    kv = ctx.new_kv_cache()
    prompts = [W.gen_prompt(wl, L0, index=b) for b in range(B)]
    # prefill: the target's hooked states of every prompt position
    toks = torch.from_numpy(np.concatenate(prompts)).to(DEV)
    hooks, nxt, _ = dfl.target_forward(twd, toks)
    ctx.inject_kv(hooks, torch.arange(B, dtype=torch.int32,
                                      device=DEV).repeat_interleave(L0),
                  torch.arange(L0, dtype=torch.int32, device=DEV).repeat(B),
                  kv)
    anchor = nxt.view(B, L0)[:, -1].contiguous()
    lens = torch.full((B,), L0, dtype=torch.int32, device=DEV)
    streams = [list(map(int, p)) for p in prompts]
    accepts = [[] for _ in range(B)]
    rng = np.random.default_rng(4)
    rounds = 0
    while min(len(s) for s in streams) < L0 + n_emit:
        draft = ctx.draft_block(lens, kv, int(lens.max()), anchor=anchor)
        if mode == "right-for-a-while":
            # the first c drafts replaced by the target's own continuation
            cuts = rng.integers(0, K, B)
            d = draft.cpu().numpy()
            t = anchor.clone()
            for j in range(int(cuts.max())):
                _, t, _ = dfl.target_forward(twd, t)
                tj = t.cpu().numpy()
                for b in range(B):
                    if j < cuts[b]:
                        d[b, j] = tj[b]
            draft = torch.from_numpy(d).to(DEV)
        block = torch.cat([anchor[:, None], draft], 1).contiguous()
        # the verify pass: the target over the whole block, its hooks kept
        hooks, tnext, _ = dfl.target_forward(twd, block.view(-1))
        acc, new_anchor = dfl.verify_greedy(draft, tnext.view(B, K))
        a = acc.cpu().numpy()
        blk = block.cpu().numpy()
        L = lens.cpu().numpy()
        # capture: the accepted positions' hooked states into the drafter
        rows = np.concatenate([b * K + np.arange(a[b]) for b in range(B)])
        ridx = torch.from_numpy(rows).to(DEV)
        ctx.inject_kv([h.index_select(0, ridx) for h in hooks],
                      torch.from_numpy(np.repeat(np.arange(B), a).astype(
                          np.int32)).to(DEV),
                      torch.from_numpy(np.concatenate(
                          [L[b] + np.arange(a[b]) for b in range(B)]).astype(
                              np.int32)).to(DEV), kv)
        for b in range(B):
            streams[b] += [int(x) for x in blk[b, :a[b]]]
            accepts[b].append(int(a[b]))
        lens += acc
        anchor = new_anchor
        rounds += 1
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    tm = TargetModel(tw)
    for b in range(B):
        n = len(streams[b]) - L0
        # the GPU target's own greedy stream, one position per launch
        t, ref = torch.tensor([prompts[b][-1]], dtype=torch.int32,
                              device=DEV), []
        for _ in range(n):
            _, t, _ = dfl.target_forward(twd, t)
            ref.append(int(t[0]))
        assert streams[b][L0:] == ref, f"seq {b}: not the target's stream"
        # every transition of the stream is the oracle target's greedy
        # choice wherever that choice is clear (a bigram target: each next
        # token depends on the previous one only)
        prev = [int(prompts[b][-1])] + streams[b][L0:-1]
        _, o_next, o_m = oracle_target(tm, prev)
        clear = o_m > MARGIN_MIN
        np.testing.assert_array_equal(np.asarray(streams[b][L0:])[clear],
                                      o_next[clear])
        say(f"  seq {b}: {n} tokens in {len(accepts[b])} rounds, accept "
            f"lengths {accepts[b]}; every transition is the oracle target's "
            f"greedy choice ({int(clear.sum())} clear, "
            f"{int((~clear).sum())} within {MARGIN_MIN} of a tie)")
    assert rounds > 3
    if mode == "right-for-a-while":
        assert max(max(x) for x in accepts) > 1
    # the oracle's own loop (its drafter, its target) emits the same stream
    # as far as the oracle target has no near tie
    model = OracleModel(wl, w_cpu)
    for b in range(B):
        y, _ = speculative_loop(model, tm, prompts[b], 32)
        k = min(len(y), len(streams[b]))
        o_stream = greedy_stream(tm, int(prompts[b][-1]), k - L0)
        _, _, m = oracle_target(tm, [int(prompts[b][-1])] + o_stream[:-1])
        ok = k - L0 if not (m <= MARGIN_MIN).any() else int(np.argmax(
            m <= MARGIN_MIN))
        assert y[:L0 + ok] == streams[b][:L0 + ok]
