"""FP8 E4M3 drafter weights on the GPU (per-output-row scales).

The kernels widen each E4M3 code to bf16 exactly (checked on every code),
run the bf16 MFMA with bf16 activations and scale each output column's sum
by its row scale.  The batch-1 paths (streaming projections, persistent LM
head) read the FP8 step pairs; batched calls run the tiled kernels on the
codes widened to bf16 at create time.  Parity against the float64 oracle of
the same codes and scales, with the float32 ensemble as the floor.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import OracleModel, draft_batch, inject_rows
from oracle.numerics import decode_e4m3
from tests.gpu_common import (DEV, Float32Floor, check_bf16_close,
                              check_single_pass, f64, say, to_dev)

pytestmark = pytest.mark.gpu

dfl = pytest.importorskip("block_diffusion_drafting_dflash_amd")


def test_fp8_widening_on_every_code():
    codes = torch.arange(256, dtype=torch.uint8).repeat(4).to(DEV)
    bits = dfl.fp8_to_bf16(codes).cpu().numpy().astype(np.uint16)
    got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = decode_e4m3(codes.cpu().numpy())
    nan = np.isnan(want)
    assert np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan], want[~nan])
    # signed zeros kept
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])
    say("[fp8] widening exact on all 256 codes")


# batch 1: streaming FP8 projections and the persistent FP8 LM head (a
# 4096-wide contraction, several vocabulary tiles per workgroup); batch 3:
# the 48-row streaming form for narrow outputs and the tiled kernels (codes
# widened) for the rest and the LM head; two passes at batch 1.
CASES = {
    "wide-fp8-b1": W.small_bf16(batch=1, hidden=4096, intermediate=2048,
                                vocab=8272, ctx_min=200, ctx_max=200,
                                name="wide-fp8-b1", seed=84,
                                weight_format="fp8"),
    "small-fp8-b1": W.small_bf16(batch=1, ctx_min=150, ctx_max=150,
                                 name="small-fp8-b1", seed=85,
                                 weight_format="fp8"),
    "small-fp8-b3": W.small_bf16(batch=3, name="small-fp8-b3", seed=86,
                                 weight_format="fp8"),
    # the persistent SwiGLU stream on FP8 pairs: 1104 gate/up tiles (four or
    # five per workgroup), a contraction of 16 pairs (one per wave)
    "ffn-fp8-b1": W.small_bf16(batch=1, num_layers=1, hidden=1024,
                               intermediate=8832, ctx_min=120, ctx_max=120,
                               name="ffn-fp8-b1", seed=97,
                               weight_format="fp8"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_step_parity(name):
    """Inject every context (prefix rows above 16 take the widened codes,
    the step's 16 rows per sequence the FP8 pairs at batch 1), draft, and
    compare K/V, logits, tokens and confidences with the oracle."""
    wl = CASES[name]
    say(f"[fp8 step] {name}")
    w_cpu = W.gen_weights(wl, random_gains=True)
    ctx = dfl.DFlash(wl, to_dev(w_cpu))
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
    kv = ctx.new_kv_cache()
    per_seq, hid_pos = [], []
    n_new = wl.new_rows
    for b, L in enumerate(lens):
        n_pre = int(L) - n_new
        hp = W.gen_hiddens(wl, n_pre, index=b, tag="prefix")
        ctx.inject_kv([h.to(DEV) for h in hp],
                      torch.full((n_pre,), b, dtype=torch.int32, device=DEV),
                      torch.arange(n_pre, dtype=torch.int32, device=DEV), kv)
    Hs = W.gen_hiddens(wl, len(lens) * n_new, tag="step")
    for b, L in enumerate(lens):  # 16 rows per call: the batch-1 form
        rows = [h[b * n_new:(b + 1) * n_new] for h in Hs]
        ctx.inject_kv([h.to(DEV) for h in rows],
                      torch.full((n_new,), b, dtype=torch.int32, device=DEV),
                      torch.arange(int(L) - n_new, int(L), dtype=torch.int32,
                                   device=DEV), kv)
    for b, L in enumerate(lens):
        hp = W.gen_hiddens(wl, int(L) - n_new, index=b, tag="prefix")
        rows = [h[b * n_new:(b + 1) * n_new] for h in Hs]
        hb = [torch.cat([a, r]) for a, r in zip(hp, rows)]
        pos = np.arange(int(L))
        per_seq.append(inject_rows(model, hb, pos))
        hid_pos.append((hb, pos))
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    for b, L in enumerate(lens):
        for l in range(wl.num_layers):
            gk = f64(kv[l, 0, b, :, :L]).transpose(1, 0, 2)
            gv = f64(kv[l, 1, b, :, :L]).transpose(1, 0, 2)
            check_bf16_close(gk, per_seq[b][l][0], f"K l{l} b{b}")
            check_bf16_close(gv, per_seq[b][l][1], f"V l{l} b{b}")
    anchors = W.gen_anchors(wl)
    B, K1 = len(lens), wl.block_size - 1
    out = {"draft": torch.full((B, K1), -7, dtype=torch.int32, device=DEV),
           "conf": torch.full((B, K1), float("nan"), device=DEV),
           "margin": torch.full((B, K1), float("nan"), device=DEV),
           "logits": torch.full((1, B, K1, wl.vocab), float("nan"),
                                device=DEV)}
    ctx.draft_block(torch.from_numpy(lens.astype(np.int32)).to(DEV), kv,
                    int(lens.max()), anchor=torch.from_numpy(anchors).to(DEV),
                    draft=out["draft"], conf=out["conf"],
                    margin=out["margin"], logits=out["logits"])
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    g = {"draft": out["draft"].cpu().numpy(),
         "conf": out["conf"].cpu().numpy(),
         "margin": out["margin"].cpu().numpy(),
         "logits_all": out["logits"].cpu().numpy().astype(np.float64)}
    ref = draft_batch(model, per_seq, lens, anchors=anchors, keep_logits=True)
    empty = {l: (np.zeros((0, wl.num_kv_heads, wl.head_dim)),) * 2
             for l in range(wl.num_layers)}
    fl = Float32Floor(wl, w_cpu, [empty] * B, lens, inject=hid_pos)
    check_single_pass(wl, name, g, ref, fl, anchors)


def test_fp8_two_passes_match_the_oracle():
    from tests.gpu_common import check_two_pass
    wl = W.small_bf16(batch=1, ctx_min=120, ctx_max=120, num_passes=2,
                      commit_per_pass=8, name="small-fp8-S2", seed=87,
                      weight_format="fp8")
    say("[fp8 S=2] small-fp8-S2")
    w_cpu = W.gen_weights(wl, random_gains=True)
    ctx = dfl.DFlash(wl, to_dev(w_cpu))
    model = OracleModel(wl, w_cpu)
    lens = W.gen_ctx_lens(wl)
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
    anchors = W.gen_anchors(wl)

    def run(block=None, S=2):
        B, K1 = len(lens), wl.block_size - 1
        o = {"draft": torch.full((B, K1), -7, dtype=torch.int32, device=DEV),
             "conf": torch.full((B, K1), float("nan"), device=DEV),
             "margin": torch.full((B, K1), float("nan"), device=DEV),
             "logits": torch.full((S, B, K1, wl.vocab), float("nan"),
                                  device=DEV)}
        ctx.draft_block(
            torch.from_numpy(lens.astype(np.int32)).to(DEV), kv,
            int(lens.max()),
            anchor=None if block is not None else
            torch.from_numpy(anchors).to(DEV),
            block_tokens=None if block is None else
            torch.from_numpy(np.asarray(block, np.int32)).to(DEV),
            num_passes=S, commit_per_pass=8 if S > 1 else 0,
            draft=o["draft"], conf=o["conf"], margin=o["margin"],
            logits=o["logits"])
        torch.cuda.synchronize()
        assert ctx.check_device_errors() == 0
        return {"draft": o["draft"].cpu().numpy(),
                "conf": o["conf"].cpu().numpy(),
                "margin": o["margin"].cpu().numpy(),
                "logits_all": o["logits"].cpu().numpy().astype(np.float64)}

    g = run()
    ref = draft_batch(model, per_seq, lens, anchors=anchors, num_passes=2,
                      commit_per_pass=8, keep_logits=True)
    fl = Float32Floor(wl, w_cpu, per_seq, lens)
    check_two_pass(wl, "small-fp8-S2", lambda blk: run(blk, 1), g, ref, fl,
                   anchors, 8)
