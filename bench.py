#!/usr/bin/env python3
"""Drafted tokens/s of one DFlash drafting step on one MI355X.

A step is the whole drafting path for one batch: KV injection of 16 new
context rows per sequence, the block draft (all layers, LM head, argmax /
confidence commit over S passes), the synthetic target's greedy tokens (a
stand-in for the target model, which is out of scope) and greedy
verification.  Inputs (weights, hidden states, ids, random draws) are resident
in HBM before the timed region; the prefix context is injected untimed.

Prints one JSON line.  `value` = drafted tokens per second = batch * (K - 1)
* steps / elapsed.  `roofline` rates the dominant kernel against its bound
(HBM bytes or MFMA flops) with its duration taken from HIP events around
each of its launches inside the timed region.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

import workloads as W

METRIC = "drafted tokens/s (K=16 block, incl. KV injection) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK = {"bf16": 2500.0, "f32": 157.3}   # dense TFLOP/s (f32: vector)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.BENCH_DEFAULT,
                    choices=list(W.WORKLOADS),
                    help="the headline workload of the JSON line")
    ap.add_argument("--only", action="store_true",
                    help="measure the headline workload only (by default "
                         "every other workload follows in `workloads`)")
    ap.add_argument("--timed-kernel", default="auto",
                    choices=["auto", "lmhead", "attention", "gemm"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged KV cache with pages of this many positions "
                         "(handed out in a shuffled order); 0: contiguous")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter scale)")
    ap.add_argument("--block-vs-one", action="store_true",
                    help="instead of the step: time the injection of 16 rows "
                         "against 1 row per sequence and a drafting pass with "
                         "15 masked positions against one with 1 (the LM "
                         "head's row count); the block-versus-step ratio of "
                         "the pages at this batch")
    ap.add_argument("--read-probe", action="store_true",
                    help="instead of the step: the HBM read rate a plain "
                         "streaming read of 1 GiB reaches (harness kernel), "
                         "the practical ceiling for the bandwidth-bound "
                         "kernels")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the step: time torch.matmul (the vendor "
                         "GEMM library) at the workload's projection and "
                         "LM-head shapes, as a reference for the MFMA "
                         "fraction the tiled kernels reach")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic cost of a step (bytes that must cross HBM, flops of the math)
# ---------------------------------------------------------------------------

def weight_bytes(wl, rows, cols):
    """Bytes of one projection matrix: the drafter dtype, or FP8 codes plus
    one float32 scale per output row."""
    if getattr(wl, "weight_format", "dtype") == "fp8":
        return rows * cols + 4 * rows
    return rows * cols * (4 if wl.dtype == "f32" else 2)


def step_cost(wl, lens):
    esz = 4 if wl.dtype == "f32" else 2
    D, I, V, d = wl.hidden, wl.intermediate, wl.vocab, wl.head_dim
    qd, kvd = wl.num_q_heads * d, wl.num_kv_heads * d
    B, K, Nl = wl.batch, wl.block_size, wl.num_layers
    T = B * wl.new_rows
    ntd = wl.num_target_layers * wl.target_hidden
    wb = lambda r, c: weight_bytes(wl, r, c)
    by = fl = 0.0
    # injection
    by += T * ntd * esz + wb(D, ntd) + Nl * wb(2 * kvd, D)
    by += T * Nl * 2 * kvd * esz + D * esz
    fl += 2.0 * T * D * ntd + 2.0 * T * Nl * 2 * kvd * D
    lm = []
    R = B * K
    for s in range(wl.num_passes):
        masked = B * (K - 1 - s * wl.commit_per_pass)
        by += R * D * esz
        layer_w = (wb(qd + 2 * kvd, D) + wb(D, qd) + wb(2 * I, D) +
                   wb(D, I) + 2 * D * esz)
        kv_read = sum((int(L) + K) * 2 * kvd * esz for L in lens)
        by += Nl * (layer_w + kv_read + R * 2 * kvd * esz)
        fl += Nl * 2.0 * R * ((qd + 2 * kvd) * D + qd * D + 3 * I * D)
        fl += Nl * sum(4.0 * wl.num_q_heads * K * (int(L) + K) * d for L in lens)
        lm_bytes = wb(V, D) + masked * D * esz + D * esz
        lm_flops = 2.0 * masked * V * D
        by += lm_bytes
        fl += lm_flops
        lm.append((lm_bytes, lm_flops))
    by += B * (2 * K - 1) * 4 * 2
    return by, fl, lm


def kernel_cost(wl, lens, kind):
    """Algorithmic (bytes, flops) per launch of the timed kernel class,
    averaged over its launches in one step."""
    esz = 4 if wl.dtype == "f32" else 2
    D, I, d = wl.hidden, wl.intermediate, wl.head_dim
    qd, kvd = wl.num_q_heads * d, wl.num_kv_heads * d
    B, K = wl.batch, wl.block_size
    if kind == "lmhead":
        _, _, lm = step_cost(wl, lens)
        return (sum(b for b, _ in lm) / len(lm), sum(f for _, f in lm) / len(lm))
    if kind == "attention":
        kv = sum((int(L) + K) * 2 * kvd * esz for L in lens)
        q_o = 2 * B * K * qd * esz
        fl = sum(4.0 * wl.num_q_heads * K * (int(L) + K) * d for L in lens)
        return kv + q_o, fl
    # every projection GEMM launch of a step: inject fc + kv, then per layer
    # qkv, o, gate/up, down
    T = B * wl.new_rows
    ntd = wl.num_target_layers * wl.target_hidden
    R = B * K
    shapes = [(T, D, ntd), (T, wl.num_layers * 2 * kvd, D)]
    for _ in range(wl.num_passes):
        for _ in range(wl.num_layers):
            shapes += [(R, qd + 2 * kvd, D), (R, D, qd), (R, 2 * I, D), (R, D, I)]
    by = sum(weight_bytes(wl, n, k) + m * k * esz for m, n, k in shapes)
    fl = sum(2.0 * m * n * k for m, n, k in shapes)
    return by / len(shapes), fl / len(shapes)


# ---------------------------------------------------------------------------

# Sources that define each timed kernel class: the LM head is the persistent
# kernel up to 16 rows and the tiled GEMM beyond; the projection GEMMs are
# the streaming or the tiled form with their shared epilogues, and a split
# GEMM's reduction (fused with the row RMSNorm that follows it where that
# norm takes its row form: epilogue.hip).
KERNEL_SOURCES = {
    "lmhead": ["gemm.hip", "gemm_tiled.hip", "gemm_epilogue.h"],
    "gemm": ["gemm.hip", "gemm_tiled.hip", "gemm_epilogue.h", "epilogue.hip"],
    "attention": ["attention.hip"],
}


def kernel_source_sha(kind):
    """sha256 over the sources that define the timed kernel."""
    import hashlib
    csrc = os.path.join(ROOT, "block_diffusion_drafting_dflash_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind] + ["common.h", "kernels.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(wl, kind):
    """HBM bytes per launch from the committed FETCH_SIZE + WRITE_SIZE
    counter summary of this kernel and workload, or None when there is none
    or the kernel's sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{wl.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_sha(kind):
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def setup(wl, torch, dfl, dev, page_size=0):
    weights = W.gen_weights(wl, device=dev)
    lens = W.gen_ctx_lens(wl)
    B, K = wl.batch, wl.block_size
    chunk = 2048
    ctx = dfl.DFlash(wl, weights, max_inject_rows=max(chunk, B * wl.new_rows))
    if page_size:
        # pages for positions [0, L_b + K) of every sequence, in a shuffled
        # order; -1 (never read) past each sequence's last page
        need = [(int(L) + K + page_size - 1) // page_size for L in lens]
        ld = (ctx.cfg.max_ctx + K + page_size - 1) // page_size
        perm = np.random.default_rng(1).permutation(sum(need))
        table = np.full((ctx.cfg.max_batch, ld), -1, dtype=np.int32)
        k = 0
        for b, n in enumerate(need):
            table[b, :n] = perm[k:k + n]
            k += n
        kv = ctx.new_kv_cache_paged(page_size, sum(need), dev)
        ctx.set_kv_pages(page_size, sum(need),
                         torch.from_numpy(table).to(dev))
    else:
        kv = ctx.new_kv_cache(dev)
    # untimed prefix: positions [0, L_b - 16) of every sequence
    prefill = None
    for b, L in enumerate(lens):
        n_pre = int(L) - wl.new_rows
        for c0 in range(0, n_pre, chunk):
            n = min(chunk, n_pre - c0)
            H = W.gen_hiddens(wl, n, device=dev, index=b * 100000 + c0 // chunk,
                              tag="prefix")
            args = (H, torch.full((n,), b, dtype=torch.int32, device=dev),
                    torch.arange(c0, c0 + n, dtype=torch.int32, device=dev))
            ctx.inject_kv(*args, kv)
            if prefill is None:
                prefill = args  # re-injected (same rows, same values) to time
    torch.cuda.synchronize()
    T = B * wl.new_rows
    inp = {
        "H": W.gen_hiddens(wl, T, device=dev, index=0, tag="step"),
        "row_seq": torch.arange(B, dtype=torch.int32,
                                device=dev).repeat_interleave(wl.new_rows),
        "row_pos": torch.from_numpy(np.concatenate(
            [np.arange(int(L) - wl.new_rows, int(L)) for L in lens]).astype(
                np.int32)).to(dev),
        "ctx_len": torch.from_numpy(lens.astype(np.int32)).to(dev),
        "anchor": torch.from_numpy(W.gen_anchors(wl)).to(dev),
    }
    inp["prefill"] = prefill
    draws = W.gen_verify_draws(wl)
    for k, v in draws.items():
        inp[k] = torch.from_numpy(v).to(dev)
    inp["draft"] = torch.zeros(B, K - 1, dtype=torch.int32, device=dev)
    inp["target"] = torch.zeros(B, K, dtype=torch.int32, device=dev)
    inp["accept"] = torch.zeros(B, dtype=torch.int32, device=dev)
    inp["next"] = torch.zeros(B, dtype=torch.int32, device=dev)
    return ctx, kv, lens, inp, weights


def make_step(ctx, kv, lens, inp, wl, torch, dfl):
    """Pre-marshalled C-ABI calls of one step on torch's current stream."""
    lib, har = dfl.load_library(), dfl.load_harness()
    vp = ctypes.c_void_p
    P = lambda t: vp(t.data_ptr())
    s = vp(torch.cuda.current_stream().cuda_stream)
    H = inp["H"]
    harr = (vp * len(H))(*[h.data_ptr() for h in H])
    hpp = ctypes.cast(harr, ctypes.POINTER(vp))
    T, ld = H[0].shape[0], H[0].stride(0)
    B, K = wl.batch, wl.block_size
    maxL = int(max(lens))
    a = dict(seq=P(inp["row_seq"]), pos=P(inp["row_pos"]), kv=P(kv),
             cl=P(inp["ctx_len"]), an=P(inp["anchor"]), dr=P(inp["draft"]),
             u=P(inp["u"]), r=P(inp["r"]), tail=P(inp["tail"]), p=P(inp["p"]),
             tg=P(inp["target"]), acc=P(inp["accept"]), nx=P(inp["next"]))
    S, c = wl.num_passes, wl.commit_per_pass
    ctxp = ctx.ctx

    def step():
        st = lib.dflash_inject_kv(ctxp, s, hpp, ld, T, a["seq"], a["pos"],
                                  a["kv"])
        st |= lib.dflash_draft_block(ctxp, s, B, a["an"], None, a["cl"], maxL,
                                     a["kv"], S, c, a["dr"], None, None, None)
        st |= har.dflash_harness_synth_target(s, B, K, wl.vocab, a["dr"],
                                              a["u"], a["r"], a["tail"],
                                              a["p"], a["tg"])
        st |= lib.dflash_verify_greedy(s, B, K, a["dr"], a["tg"], a["acc"],
                                       a["nx"])
        if st != 0:
            raise RuntimeError("a drafting call failed: " +
                               lib.dflash_last_error().decode())
    return step


def cpu_baseline(wl, weights, lens, budget_s):
    """The oracle as it stands, one step at a time on a sample of the
    workload's sequences: inject the 16 new rows, draft, verify."""
    import torch
    from oracle import (OracleModel, draft_batch, inject_rows,
                        synthetic_target, verify_greedy)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or
                      [1])
    except Exception:
        threads = os.cpu_count() or 1
    model = OracleModel(wl, weights)
    draws = W.gen_verify_draws(wl)
    anchors = W.gen_anchors(wl)
    H_step = W.gen_hiddens(wl, wl.batch * wl.new_rows, device="cuda", index=0,
                           tag="step")
    H_step = [h.cpu() for h in H_step]
    n_new = wl.new_rows
    done_seqs, elapsed, steps = 0, 0.0, 0
    b = 0
    while elapsed < budget_s and steps < 64:
        L = int(lens[b])
        # context prefix: seeded stand-in with the injected prefix's shape
        prefix = {}
        for l in range(wl.num_layers):
            k = W.gen_kv_prefix(wl, l, "k", b, L - n_new).float().numpy()
            v = W.gen_kv_prefix(wl, l, "v", b, L - n_new).float().numpy()
            prefix[l] = (k.astype(np.float64).transpose(1, 0, 2),
                         v.astype(np.float64).transpose(1, 0, 2))
        rows = slice(b * n_new, (b + 1) * n_new)
        t0 = time.perf_counter()
        new = inject_rows(model, [h[rows] for h in H_step],
                          np.arange(L - n_new, L))
        ctx_kv = {l: (np.concatenate([prefix[l][0], new[l][0]]),
                      np.concatenate([prefix[l][1], new[l][1]]))
                  for l in model.layers}
        res = draft_batch(model, [ctx_kv], [L], anchors=[anchors[b]],
                          num_passes=wl.num_passes,
                          commit_per_pass=wl.commit_per_pass)[0]
        Tg = synthetic_target(res["draft"][None], draws["u"][b:b + 1],
                              draws["r"][b:b + 1], draws["tail"][b:b + 1],
                              draws["p"], wl.vocab)
        verify_greedy(res["draft"], Tg[0])
        elapsed += time.perf_counter() - t0
        steps += 1
        done_seqs += 1
        b = (b + 1) % wl.batch
    return {"value": done_seqs * (wl.block_size - 1) / elapsed,
            "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{steps} single-sequence step(s) of {wl.name} "
                       f"(inject 16 rows + {wl.num_passes}-pass draft + "
                       f"verify; context prefix from the seeded generator), "
                       f"{elapsed:.1f} s of float64 numpy on the host")}


def auto_kernel(wl):
    """The kernel class that dominates a workload's step."""
    return {"qwen3-8b-3L-b4-ctx32k": "attention",
            "qwen3-8b-3L-b64-ctx256-2k-S2": "gemm",
            "qwen3-8b-5L-b16-ctx1k-4k": "gemm"}.get(wl.name, "lmhead")


def measure(wl, args, torch, dfl, dev, kind, full=True):
    """Time one workload: exactly args.steps steps after args.warmup, then
    the same steps with dispatch-bound events on the timed kernel class,
    then with one event per step boundary.  Returns (entry, extras)."""
    ctx, kv, lens, inp, weights = setup(wl, torch, dfl, dev, args.page_size)
    step = make_step(ctx, kv, lens, inp, wl, torch, dfl)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if ctx.check_device_errors() != 0:
        raise RuntimeError("device error during warmup")

    # Timed region: exactly K steps, bracketed by synchronisation, with no
    # instrumentation inside (an event bound to a kernel dispatch holds the
    # stream for a few microseconds on either side of that kernel).
    run = step
    graph = None
    if args.graph:
        # the step's launches captured once (the calls enqueue kernels only);
        # the step closure binds the stream that is current when it is made
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            make_step(ctx, kv, lens, inp, wl, torch, dfl)()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            make_step(ctx, kv, lens, inp, wl, torch, dfl)()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            run()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(
        enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        run()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    # Kernel region: the same K steps again, with HIP events bound to every
    # launch of the timed kernel class on its launch stream.
    ctx.set_kernel_timing(kind)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total_ev = t0.elapsed_time(t1)
    n_launch, k_ms = ctx.kernel_timing()
    ctx.set_kernel_timing("off")
    # Step-time spread: the same steps with one event at each step boundary.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        run()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1])
                         for i in range(args.steps)])
    extras = {}
    if full:
        # Host cost of issuing one step (the calls only enqueue work): each
        # step is issued onto an idle stream, timed on the host clock until
        # the calls return, then synchronised.
        host_us = []
        for _ in range(min(args.steps, 20)):
            torch.cuda.synchronize()
            h0 = time.perf_counter()
            run()
            host_us.append((time.perf_counter() - h0) * 1e6)
        torch.cuda.synchronize()
        extras["host_enqueue_us_per_step"] = round(float(np.median(host_us)),
                                                   1)
        # Injection of a whole context chunk (the untimed set-up's first
        # call, repeated with the same rows and values).
        prefill = None
        if inp["prefill"] is not None:
            H, seq, pos = inp["prefill"]
            ctx.inject_kv(H, seq, pos, kv)
            torch.cuda.synchronize()
            t0.record(stream)
            ctx.inject_kv(H, seq, pos, kv)
            t1.record(stream)
            torch.cuda.synchronize()
            pf_ms = t0.elapsed_time(t1)
            prefill = {"rows": int(seq.numel()), "ms": round(pf_ms, 4),
                       "rows_per_s": round(seq.numel() / (pf_ms / 1e3), 1)}
        extras["prefill_inject"] = prefill
    if ctx.check_device_errors() != 0:
        raise RuntimeError("device error during the timed steps")
    ms_step = ms_total / args.steps
    drafted = wl.batch * (wl.block_size - 1)
    value = drafted * args.steps / (ms_total / 1e3)

    by, fl, _ = step_cost(wl, lens)
    kb, kf = kernel_cost(wl, lens, kind)
    k_avg_s = (k_ms / max(n_launch, 1)) / 1e3
    bound = "hbm" if (kf / max(kb, 1)) < (MFMA_PEAK[wl.dtype] * 1e12 /
                                          (HBM_PEAK_GBS * 1e9)) else "mfma"
    if bound == "hbm":
        ach, peak, unit = kb / k_avg_s / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        ach, peak, unit = kf / k_avg_s / 1e12, MFMA_PEAK[wl.dtype], "TFLOP/s"
    acc = inp["accept"].cpu().numpy()
    K = wl.block_size
    p10, p50, p90 = (float(np.percentile(per_step, q)) for q in (10, 50, 90))
    entry = {
        "workload": wl.name, "dtype": wl.dtype,
        "weights": ("fp8-e4m3, per-row fp32 scales" if wl.weight_format ==
                    "fp8" else wl.dtype),
        "config": {"workload": wl.name, "batch": wl.batch,
                   "ctx_len": [int(lens.min()), int(lens.max())],
                   "block": K, "draft_layers": wl.num_layers,
                   "passes": wl.num_passes,
                   "commit_per_pass": wl.commit_per_pass,
                   "new_rows_per_seq": wl.new_rows,
                   "launch": "hip_graph" if args.graph else "stream",
                   "kv_cache": (f"paged-{args.page_size}" if args.page_size
                                else "contiguous")},
        "value": round(value, 1), "ms_per_step": round(ms_step, 5),
        "step_ms_p10_p50_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
        "tokens_per_s_at_median_step": round(drafted / (p50 / 1e3), 1),
        "block_rows_per_s": round(wl.batch * K * args.steps /
                                  (ms_total / 1e3), 1),
        "accepted_tokens_per_s": round(float(acc.sum()) * args.steps /
                                       (ms_total / 1e3), 1),
        "roofline": {"kernel": kind, "bound": bound, "achieved": round(ach, 1),
                     "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                     "traffic": measured_traffic(wl, kind),
                     "launches": n_launch,
                     "avg_us": round(k_avg_s * 1e6, 2),
                     "timed_in": "a second pass of the same K steps with "
                                 "dispatch-bound HIP events on this kernel "
                                 "class",
                     "ms_per_step_with_events": round(
                         ms_total_ev / args.steps, 5),
                     "alg_bytes_per_launch": int(kb),
                     "alg_flops_per_launch": kf},
        "step": {"alg_bytes": int(by), "alg_flops": fl,
                 "hbm_frac": round(by / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                                   4),
                 "mfma_frac": round(fl / (ms_step / 1e3) / 1e12 /
                                    MFMA_PEAK[wl.dtype], 4),
                 "mean_accept_len": float(acc.mean()),
                 # accept length a = tau + 1 in [1, K]; drafts wasted per
                 # sequence-step = (K - 1) - tau
                 "accept_len_hist": np.bincount(acc, minlength=K + 1)[
                     1:].astype(int).tolist(),
                 "drafts_wasted_per_seq_step": float(
                     ((K - 1) - (acc - 1)).mean())},
    }
    del ctx, kv, inp, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry, extras, weights, lens


def vendor_gemm(wl, torch, dev, reps=10):
    """Median time of torch.matmul(A, W^T) in the drafter dtype at the
    shapes of one batched step's GEMMs (A: rows x K, W: N x K as stored)."""
    B, K = wl.batch, wl.block_size
    D, I, V, d = wl.hidden, wl.intermediate, wl.vocab, wl.head_dim
    qd, kvd = wl.num_q_heads * d, wl.num_kv_heads * d
    R = B * K
    shapes = [("qkv", R, D, qd + 2 * kvd), ("o", R, qd, D),
              ("gate_up", R, D, 2 * I), ("down", R, I, D),
              ("fc", B * wl.new_rows, wl.num_target_layers * wl.target_hidden,
               D),
              ("lm_head", B * (K - 1), D, V)]
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    peak = MFMA_PEAK["f32" if wl.dtype == "f32" else "bf16"]
    out = []
    for name, m, k, n in shapes:
        a = torch.randn(m, k, device=dev, dtype=dt)
        w = torch.randn(n, k, device=dev, dtype=dt)
        for _ in range(3):
            torch.matmul(a, w.t())
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, w.t())
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        us = ts[len(ts) // 2]
        tf = 2.0 * m * n * k / us / 1e6
        out.append({"gemm": name, "m": m, "k": k, "n": n, "us": round(us, 2),
                    "tflops": round(tf, 1), "frac": round(tf / peak, 4)})
        print(f"# {name} {m}x{k}x{n}: {us:.1f} us, {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del a, w
    return {"vendor_gemm": out, "workload": wl.name,
            "library": "torch.matmul (hipBLASLt)", "peak_tflops": peak,
            "timing": f"median of {reps} calls, HIP events"}


def read_probe(torch, dfl, dev, reps=5):
    """Median time of the harness's plain streaming read of 1 GiB at several
    grid sizes (16 waves per workgroup, 8 KiB per wave in flight)."""
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = []
    for grid in (256, 512, 1024, 2048):
        dfl.read_probe(buf, grid, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            dfl.read_probe(buf, grid, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        us = ts[len(ts) // 2]
        gbs = nbytes / us / 1e3
        out.append({"grid": grid, "us": round(us, 1), "GB/s": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
        print(f"# read probe grid {grid}: {us:.1f} us, {gbs:.1f} GB/s",
              file=sys.stderr, flush=True)
    return {"read_probe": out, "bytes": nbytes, "peak_GBs": HBM_PEAK_GBS,
            "timing": f"median of {reps} calls, HIP events"}


def block_vs_one(wl, torch, dfl, dev, reps=30):
    """The pages compare one K-token block pass with one single-token draft
    step.  The library drafts K = 16 positions per pass, so the parts whose
    cost depends on the row count are timed at both sizes: the injection of
    the new context rows (fc and the K/V projections: 16 rows per sequence
    against 1) and the drafting pass with 15 masked positions against a pass
    whose block gives 14 of them (one masked position: one LM-head row per
    sequence; the layers still run the 16 block rows)."""
    ctx, kv, lens, inp, weights = setup(wl, torch, dfl, dev)
    B, K = wl.batch, wl.block_size
    maxL = int(max(lens))
    last = torch.arange(B, device=dev) * wl.new_rows + wl.new_rows - 1
    H1 = [h.index_select(0, last).contiguous() for h in inp["H"]]
    seq1 = inp["row_seq"].index_select(0, last).contiguous()
    pos1 = inp["row_pos"].index_select(0, last).contiguous()
    rng = np.random.default_rng(11)
    blk = rng.integers(0, wl.vocab - 1, (B, K)).astype(np.int32)
    blk[:, 0] = inp["anchor"].cpu().numpy()
    blk[:, K - 1] = wl.mask_id
    blk = torch.from_numpy(blk).to(dev)
    draft = torch.zeros(B, K - 1, dtype=torch.int32, device=dev)
    cases = {
        "inject_16_rows": lambda: ctx.inject_kv(
            inp["H"], inp["row_seq"], inp["row_pos"], kv),
        "inject_1_row": lambda: ctx.inject_kv(H1, seq1, pos1, kv),
        "draft_pass_15_masked": lambda: ctx.draft_block(
            inp["ctx_len"], kv, maxL, anchor=inp["anchor"], draft=draft),
        "draft_pass_1_masked": lambda: ctx.draft_block(
            inp["ctx_len"], kv, maxL, block_tokens=blk, draft=draft),
    }
    out = {}
    for name, fn in cases.items():
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        out[name + "_ms"] = round(ts[len(ts) // 2], 5)
        print(f"# {name}: {out[name + '_ms']} ms", file=sys.stderr, flush=True)
    if ctx.check_device_errors() != 0:
        raise RuntimeError("device error in the block-versus-one runs")
    t16 = out["inject_16_rows_ms"] + out["draft_pass_15_masked_ms"]
    t1 = out["inject_1_row_ms"] + out["draft_pass_1_masked_ms"]
    out["block_over_one"] = round(t16 / t1, 4)
    return {"block_vs_one": out, "workload": wl.name,
            "timing": f"median of {reps} calls, HIP events"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the drafting path runs on one GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_drafting_dflash_amd as dfl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.workload]
    if args.vendor_gemm:
        print(json.dumps(vendor_gemm(wl, torch, dev)), flush=True)
        return
    if args.read_probe:
        print(json.dumps(read_probe(torch, dfl, dev)), flush=True)
        return
    if args.block_vs_one:
        print(json.dumps(block_vs_one(wl, torch, dfl, dev)), flush=True)
        return
    kind = args.timed_kernel if args.timed_kernel != "auto" else auto_kernel(wl)
    head, extras, weights, lens = measure(wl, args, torch, dfl, dev, kind)
    print(f"# {wl.name}: {head['ms_per_step']} ms/step, {head['value']} "
          f"tokens/s", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"],
        "tokens_per_s_at_median_step": head["tokens_per_s_at_median_step"],
        "block_rows_per_s": head["block_rows_per_s"],
        "accepted_tokens_per_s": head["accepted_tokens_per_s"],
    }
    out.update(extras)
    out["step"] = head["step"]
    if args.copy_calibration:
        n = 1 << 28
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
        del a, b
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(wl, weights, lens, args.cpu_budget)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 3)
    del weights
    torch.cuda.empty_cache()
    if not args.only:
        rest = []
        for name in W.WORKLOAD_ORDER + W.EXTRA_WORKLOADS:
            if name == wl.name:
                continue
            w2 = W.WORKLOADS[name]
            e, _, wts, _ = measure(w2, args, torch, dfl, dev, auto_kernel(w2),
                                   full=False)
            del wts
            torch.cuda.empty_cache()
            print(f"# {name}: {e['ms_per_step']} ms/step, {e['value']} "
                  f"tokens/s", file=sys.stderr, flush=True)
            rest.append(e)
        out["workloads"] = rest
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
