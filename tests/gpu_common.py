"""Helpers shared by the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import sys
from typing import Dict, List

import numpy as np
import torch

import workloads as W
from oracle import OracleModel, inject_rows, round_bf16
from tests import floor_eval

DEV = "cuda"

# Tolerances.  The stated bounds: logits max-abs 2e-2 (bf16, float32
# accumulation) or 1e-4 (f32 drafter); log-confidence 4e-2 / 2e-4; token ids
# exact wherever the oracle's top-2 margin exceeds 1e-2.
#
# A bf16 drafter stores its activations in bf16 at eight points per layer.
# Float32 sums decide a few of those roundings differently from the float64
# oracle, and every such flip moves whole rows of the next projection, which
# the next norm and MLP spread over the hidden state: an exact float32
# evaluation of the same step (tests/floor_eval.py) lands about 2e-2 from the
# oracle at one Qwen3-8B-shaped layer and 5e-2 at five.  So for bf16 the
# logit (and log-confidence) bound is max(stated, 1.25 x floor), where the
# floor is the largest distance from the oracle of an ensemble of float32
# evaluations of the very inputs of the test (each summing the projections'
# contractions in a different seeded order), and a token that differs from
# the oracle's where its margin exceeds 1e-2 is accepted only if some member
# of that ensemble also differs there: float32 arithmetic demonstrably
# decides it either way.  Every such acceptance is counted and printed.
STATED_LOGIT = {"bf16": 2e-2, "f32": 1e-4}
STATED_LOGCONF = {"bf16": 4e-2, "f32": 2e-4}
MARGIN_MIN = 1e-2
FLOOR_FACTOR = 1.25
ENSEMBLE = 8


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(w: Dict[str, object], device=DEV):
    out = {}
    for k, v in w.items():
        out[k] = [t.to(device) for t in v] if isinstance(v, list) else v.to(device)
    return out


def f64(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_bf16_close(gpu, ref, what="", rel_rms=1e-2):
    """bf16 tensors computed from bf16-stored intermediates.

    The stored intermediate (e.g. H_cond) is rounded to bf16 from an fp32
    value on the GPU and an fp64 value in the oracle; about 1e-3 of its
    elements land on neighbouring bf16 values, and each such flip moves every
    element computed from that row by |W_ij| * ulp(c_j), an absolute amount.
    Worst case at these shapes: |c_j| up to ~4.5 (unit-RMS features times
    gains up to 1.5) has ulp 2^-5, |W_ij| up to 4 sigma = 0.08, and RoPE adds
    two such terms: ~5e-3, about 1% of RMS(K) ~ 0.46.  So:
    |gpu - ref| <= 1 ulp(max magnitude) + rel_rms * RMS(ref), and at least
    99% of elements within 1 ulp (the common case stays tight).
    """
    gpu, ref = np.asarray(gpu), np.asarray(ref)
    np.testing.assert_array_equal(round_bf16(gpu), gpu)  # stored as bf16
    ulp = bf16_ulp(np.maximum(np.abs(gpu), np.abs(ref)))
    err = np.abs(gpu - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = ulp + rel_rms * rms
    worst = float((err / bound).max())
    frac1 = float(np.mean(err <= ulp))
    assert worst <= 1.0, (f"{what}: error {err.max():.3e} exceeds 1 ulp + "
                          f"{rel_rms} * rms ({rms:.3e}) by {worst:.2f}x")
    assert frac1 >= 0.99, f"{what}: only {frac1:.5f} within 1 ulp"
    return worst, frac1


def cache_rows(kv: torch.Tensor, l: int, b: int, L: int):
    """(K [L, Hkv, d], V [L, Hkv, d]) float64 from a GPU cache tensor."""
    k = f64(kv[l, 0, b, :, :L, :]).transpose(1, 0, 2)
    v = f64(kv[l, 1, b, :, :L, :]).transpose(1, 0, 2)
    return k, v


def oracle_inject_sequence(model: OracleModel, wl, hid_chunks, pos):
    """Oracle injection of one sequence's rows: {layer: (K, V)}."""
    return inject_rows(model, hid_chunks, pos)


class Float32Floor:
    """The float32 ensemble (tests/floor_eval.py) on one test's inputs.

    ctx[j]: {layer: (K [L, Hkv, d], V)} context of sampled sequence j that
    both sides take as data; inject[j]: None or (hiddens, positions) of rows
    each member injects itself after that context (as the GPU and the
    oracle do).  lens[j]: the context length of sequence j.  f32 drafters
    store nothing in bf16: no ensemble, the stated bounds apply."""

    def __init__(self, wl, w_cpu, ctx, lens, inject=None, members=ENSEMBLE):
        self.wl = wl
        self.on = wl.dtype == "bf16"
        self.members = members if self.on else 0
        self.lens = [int(L) for L in lens]
        self.ctx = [{l: (torch.from_numpy(np.ascontiguousarray(k)).float(),
                         torch.from_numpy(np.ascontiguousarray(v)).float())
                     for l, (k, v) in c.items()} for c in ctx]
        if not self.on:
            return
        self.p = floor_eval.Prepared(wl, w_cpu, torch.float32)
        self.new = [[None] * len(ctx) for _ in range(self.members)]
        if inject is not None:
            for m in range(self.members):
                for j, inj in enumerate(inject):
                    if inj is not None:
                        self.new[m][j] = floor_eval.inject(self.p, inj[0],
                                                           inj[1], m)

    def _ctx(self, m, j):
        c, new = self.ctx[j], self.new[m][j]
        if new is None:
            return c
        return {l: (torch.cat([c[l][0], torch.from_numpy(new[l][0]).float()]),
                    torch.cat([c[l][1], torch.from_numpy(new[l][1]).float()]))
                for l in c}

    def injected(self, m, j):
        return self.new[m][j]

    def logits(self, blocks):
        """blocks[j]: block tokens [K] (mask id = masked) per sequence ->
        out[m][j] = logits [masked rows, V] of member m."""
        out = []
        for m in range(self.members):
            out.append([floor_eval.pass_logits(self.p, self._ctx(m, j),
                                               self.lens[j], blocks[j], m)[1]
                        for j in range(len(blocks))])
        return out


def logit_bound(wl, floor: float) -> float:
    if wl.dtype != "bf16":
        return STATED_LOGIT[wl.dtype]
    return max(STATED_LOGIT["bf16"], FLOOR_FACTOR * floor)


def logconf_bound(wl, floor: float) -> float:
    if wl.dtype != "bf16":
        return STATED_LOGCONF[wl.dtype]
    return max(STATED_LOGCONF["bf16"], FLOOR_FACTOR * floor)


def _logconf(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max(1)
    return -np.log(np.exp(z - m[:, None]).sum(1))


def check_pass(wl, label, items):
    """Logit, token and log-confidence parity of one pass.

    items: one dict per sequence -- rows (block indices), z_gpu [n, V],
    tok_gpu [n], z_or [n, V], tok_or [n], margin_or [n], members: list of
    member logits [n, V] (empty for f32), conf_gpu [n] or None.  Asserts the
    bounds above and returns the counts."""
    floor = lf = 0.0
    for it in items:
        zo = it["z_or"]
        for zm in it["members"]:
            floor = max(floor, float(np.abs(zm - zo).max()))
            lf = max(lf, float(np.abs(_logconf(zm) - _logconf(zo)).max()))
    bound, lbound = logit_bound(wl, floor), logconf_bound(wl, lf)
    st = {"compared": 0, "excluded": 0, "witnessed": 0, "max_dl": 0.0,
          "floor": floor, "bound": bound, "max_dlc": 0.0, "lc_bound": lbound}
    for j, it in enumerate(items):
        dl = float(np.abs(it["z_gpu"] - it["z_or"]).max())
        st["max_dl"] = max(st["max_dl"], dl)
        assert dl <= bound, (f"{label} seq {j}: logits max-abs diff {dl:.3e} > "
                             f"{bound:.3e} (float32 floor {floor:.3e})")
        if it.get("conf_gpu") is not None:
            dlc = float(np.abs(np.log(it["conf_gpu"]) -
                               _logconf(it["z_or"])).max())
            st["max_dlc"] = max(st["max_dlc"], dlc)
            assert dlc <= lbound, (f"{label} seq {j}: log-confidence diff "
                                   f"{dlc:.3e} > {lbound:.3e}")
        for r in range(len(it["rows"])):
            if it["margin_or"][r] <= MARGIN_MIN:
                st["excluded"] += 1
                continue
            st["compared"] += 1
            if it["tok_gpu"][r] == it["tok_or"][r]:
                continue
            flipped = [int(zm[r].argmax()) for zm in it["members"]
                       if int(zm[r].argmax()) != it["tok_or"][r]]
            assert flipped, (
                f"{label} seq {j} pos {it['rows'][r]}: token "
                f"{it['tok_gpu'][r]} vs {it['tok_or'][r]} (margin "
                f"{it['margin_or'][r]:.3e}); no float32 evaluation differs")
            st["witnessed"] += 1
    say(f"  {label}: max |dlogit| {st['max_dl']:.2e} (float32 floor "
        f"{floor:.2e}, bound {bound:.2e}); max |dlogconf| "
        f"{st['max_dlc']:.2e} (bound {lbound:.2e}); tokens compared "
        f"{st['compared']}, near ties {st['excluded']}, mismatches "
        f"witnessed by float32 {st['witnessed']}")
    return st


def pass_items(g_logits, g_draft, g_conf, ref, pass_idx, members=None,
               seqs=None):
    """check_pass items for pass pass_idx from GPU arrays (indexed like
    ref) and the oracle's draft_sequence results; members[m][j] logits."""
    items = []
    for j, o in enumerate(ref):
        rows = np.asarray(o["masked_rows"][pass_idx])
        zo = o["logits"][pass_idx]
        items.append({
            "rows": rows,
            "z_gpu": g_logits[j][rows - 1],
            "tok_gpu": g_draft[j][rows - 1],
            "z_or": zo,
            "tok_or": np.array([o["pass_token"][pass_idx][int(i)]
                                for i in rows]),
            "margin_or": np.array([o["pass_margin"][pass_idx][int(i)]
                                   for i in rows]),
            "members": [] if members is None else [mz[j] for mz in members],
            "conf_gpu": None if g_conf is None else g_conf[j][rows - 1],
        })
    return items


def anchor_blocks(wl, anchors):
    out = []
    for a in anchors:
        blk = np.full(wl.block_size, wl.mask_id, dtype=np.int64)
        blk[0] = int(a)
        out.append(blk)
    return out


def check_single_pass(wl, label, g, ref, fl, anchors):
    """Pass-1 logits, tokens, log-confidences and margins of every
    sequence against the oracle, with the float32 ensemble as the floor."""
    members = fl.logits(anchor_blocks(wl, anchors)) if fl.on else None
    st = check_pass(wl, label, pass_items(g["logits_all"][0], g["draft"],
                                          g["conf"], ref, 0, members))
    assert st["compared"] > 0
    mg = np.stack([o["margin"][1:] for o in ref])
    assert np.abs(g["margin"] - mg).max() <= 2 * st["bound"]
    return st


def commit_set(conf, c):
    """Block indices of the c most confident masked positions (ties ->
    lower index), from confidences of positions 1..15 (nan = committed)."""
    idx = [i for i in range(15) if not np.isnan(conf[i])]
    order = sorted(idx, key=lambda i: (-conf[i], i))
    return set(int(i) + 1 for i in order[:c])


def check_two_pass(wl, label, draft_fn, g, ref, fl, anchors, c, seqs=None):
    """S = 2 parity.  Pass 1 as a single pass; the pass-1 commit set where
    the oracle's cut is clear (an unclear cut or a differing set must be
    witnessed by a float32 evaluation); pass 2 from the GPU's own commits
    where they equal the oracle's; then pass 2 teacher-forced from the
    oracle's commits (the caller-given block) for every sequence.  g and
    ref are indexed like seqs (default: all); draft_fn(blocks [B, K]) runs
    one GPU pass over the whole batch and returns arrays indexed like seqs.
    Returns the teacher blocks (indexed by sequence)."""
    seqs = list(range(len(ref))) if seqs is None else list(seqs)
    blocks1 = anchor_blocks(wl, [anchors[b] for b in seqs])
    m1 = fl.logits(blocks1) if fl.on else None
    items1 = pass_items(g["logits_all"][0], g["draft"], None, ref, 0, m1)
    for j, it in enumerate(items1):
        # the returned id of a position committed in pass 2 is its pass-2
        # id; its pass-1 argmax is read from the pass-1 logits
        p2 = ~np.isnan(g["logits_all"][1][j][it["rows"] - 1, 0])
        it["tok_gpu"] = np.where(p2, it["z_gpu"].argmax(1), it["tok_gpu"])
    st1 = check_pass(wl, f"{label} pass 1", items1)
    teacher = [t.copy() for t in anchor_blocks(wl, anchors)]
    same_items, clear, witnessed, n_cm = [], 0, 0, 0
    for j, (b, o) in enumerate(zip(seqs, ref)):
        c1 = o["pass_conf"][0][1:]
        order = sorted(range(15), key=lambda i: (-c1[i], i))
        gap = np.log(c1[order[c - 1]]) - np.log(c1[order[c]])
        oracle_set = set(np.nonzero(o["pass"] == 0)[0].tolist())
        gpu_set = set(range(1, 16)) - set(
            np.nonzero(~np.isnan(g["logits_all"][1][j][:, 0]))[0] + 1)
        member_sets = []
        for mz in (m1 or []):
            conf = np.full(15, np.nan)
            conf[np.asarray(o["masked_rows"][0]) - 1] = np.exp(
                -np.log(np.exp(mz[j] - mz[j].max(1)[:, None]).sum(1)))
            member_sets.append(commit_set(conf, c))
        if gpu_set != oracle_set:
            assert gap <= MARGIN_MIN or any(
                ms != oracle_set for ms in member_sets), (
                f"{label} seq {b}: commit sets differ at a clear cut "
                f"(log-conf gap {gap:.3e}) that no float32 evaluation moves")
            witnessed += 1
        else:
            clear += 1
            same = all(g["draft"][j, i - 1] == o["tokens"][i]
                       for i in oracle_set)
            # the confidence and margin returned for the pass-1 commits
            for i in oracle_set:
                if g["draft"][j, i - 1] != o["tokens"][i]:
                    continue
                n_cm += 1
                dlc = abs(np.log(g["conf"][j, i - 1]) - np.log(o["conf"][i]))
                assert dlc <= st1["lc_bound"], (
                    f"{label} seq {b} pos {i}: returned log-confidence "
                    f"differs by {dlc:.3e}")
                dm = abs(g["margin"][j, i - 1] - o["margin"][i])
                assert dm <= 2 * st1["bound"], (
                    f"{label} seq {b} pos {i}: returned margin differs by "
                    f"{dm:.3e}")
            if same:  # pass 2 starts from the oracle's block
                rows2 = np.asarray(o["masked_rows"][1])
                same_items.append({
                    "rows": rows2, "z_gpu": g["logits_all"][1][j][rows2 - 1],
                    "tok_gpu": g["draft"][j][rows2 - 1],
                    "z_or": o["logits"][1],
                    "tok_or": np.array([o["pass_token"][1][int(i)]
                                        for i in rows2]),
                    "margin_or": np.array([o["pass_margin"][1][int(i)]
                                           for i in rows2]),
                    "members": [], "conf_gpu": None, "seq": j})
        for i in oracle_set:
            teacher[b][i] = o["tokens"][i]
    say(f"  {label}: pass-1 commit sets equal {clear} of {len(seqs)}, "
        f"differing (witnessed or unclear cut) {witnessed}; returned "
        f"confidence and margin of pass-1 commits compared at {n_cm} "
        f"positions")
    # second pass teacher-forced with the oracle's pass-1 commits (other
    # sequences draft a fresh block in the same launch)
    tf = draft_fn(np.stack(teacher))
    m2 = fl.logits([teacher[b] for b in seqs]) if fl.on else None
    check_pass(wl, f"{label} pass 2 (teacher-forced)", pass_items(
        tf["logits_all"][0], tf["draft"], tf["conf"], ref, 1, m2))
    if same_items:
        for it in same_items:
            it["members"] = [mz[it["seq"]] for mz in (m2 or [])]
        check_pass(wl, f"{label} pass 2 (own commits)", same_items)
    return teacher


def kv_flip_stats(gpu, ref, members, what, quiet=False):
    """Injected K/V against the oracle in bf16 ulps, next to the float32
    evaluations' own injections; returns (GPU, worst member) statistics as
    (fraction exact, fraction within 1 ulp, max |error| / ulp)."""
    def st(x):
        ulp = bf16_ulp(np.maximum(np.abs(x), np.abs(ref)))
        e = np.abs(x - ref) / ulp
        return float(np.mean(e == 0)), float(np.mean(e <= 1)), float(e.max())
    g = st(gpu)
    ms = [st(m) for m in members]
    worst = (min(m[0] for m in ms), min(m[1] for m in ms),
             max(m[2] for m in ms)) if ms else None
    ga = float(np.abs(gpu - ref).max())
    ma = max((float(np.abs(m - ref).max()) for m in members), default=0.0)
    if not quiet:
        say(f"  {what}: GPU exact {g[0]:.5f}, within 1 ulp {g[1]:.5f}, max "
            f"{g[2]:.1f} ulp ({ga:.2e}); float32 evaluations (worst) exact "
            f"{worst[0]:.5f}, within 1 ulp {worst[1]:.5f}, max "
            f"{worst[2]:.1f} ulp ({ma:.2e})" if worst else
            f"  {what}: GPU exact {g[0]:.5f}, within 1 ulp {g[1]:.5f}")
    return g, worst
