"""Helpers shared by the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import sys
from typing import Dict, List

import numpy as np
import torch

import workloads as W
from oracle import OracleModel, inject_rows, round_bf16

DEV = "cuda"

# Tolerances: logits max-abs 2e-2 (bf16, fp32 accumulate) / 1e-4 (f32);
# token ids compared where the oracle's top-2 margin exceeds 1e-2.  These
# hold as they are for a one-layer drafter.  Every further layer adds eight
# bf16 rounding points whose rare disagreements between two correct
# implementations are amplified by the next normalisation and MLP, so the
# bounds scale with the number of draft layers: an exact float32 evaluation
# of the same computation (tests/precision_floor.py) already lands 1.8e-2 to
# 2.4e-2 from the float64 oracle for a two-layer drafter of hidden size 4096,
# and 3.4e-2 / 4.5e-2 for three / five layers at Qwen3-8B shapes.
LOGIT_TOL = {"bf16": 2e-2, "f32": 1e-4}
LOGCONF_TOL = {"bf16": 4e-2, "f32": 2e-4}
MARGIN_MIN = 1e-2


def logit_tol(wl) -> float:
    return LOGIT_TOL[wl.dtype] * wl.num_layers


def logconf_tol(wl) -> float:
    return LOGCONF_TOL[wl.dtype] * wl.num_layers


def margin_min(wl) -> float:
    return MARGIN_MIN * wl.num_layers


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


def compare_draft(wl, gpu_res, oracle_res, rows_per_seq=None, tol=None,
                  margin_min=None):
    """Token / logit / confidence parity for one pass.

    gpu_res: dict of numpy arrays draft [B, K-1], conf, margin, logits
    [B, K-1, V] (rows computed in this pass); oracle_res: list of
    draft_sequence results.  Returns counts of compared / excluded tokens.
    """
    tol = logit_tol(wl) if tol is None else tol
    margin_min = globals()["margin_min"](wl) if margin_min is None else margin_min
    compared = excluded = 0
    max_dl = 0.0
    for b, o in enumerate(oracle_res):
        rows = o["masked_rows"][0]
        z = o["logits"][0]
        zg = gpu_res["logits"][b, rows - 1, :]
        dl = np.abs(zg - z).max()
        max_dl = max(max_dl, float(dl))
        assert dl <= tol, f"seq {b}: logits max-abs diff {dl:.3e} > {tol}"
        for j, i in enumerate(rows):
            m = o["pass_margin"][0][int(i)]
            if m > margin_min:
                compared += 1
                assert gpu_res["draft"][b, i - 1] == o["pass_token"][0][int(i)], (
                    f"seq {b} pos {i}: token {gpu_res['draft'][b, i - 1]} vs "
                    f"{o['pass_token'][0][int(i)]} (margin {m:.3e})")
            else:
                excluded += 1
    return compared, excluded, max_dl
