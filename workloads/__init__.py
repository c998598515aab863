"""Seeded synthetic workloads for the DFlash drafting step.

This module only *generates inputs*: drafter shapes, random weights, target
hidden states, anchors, context lengths and the random draws of the synthetic
target.  It holds none of the method's arithmetic, so both the HIP path and the
CPU oracle can take their inputs from it without sharing any computation.

Values follow the workloads the pages imply: weights N(0, 0.02), target hidden
states N(0, 1), RMSNorm gains 1.0, anchor ids uniform over the vocabulary minus
the mask id (the last id).  bf16 workloads round every generated tensor to bf16
(round to nearest even, done by torch's dtype conversion) before either side
sees it, so both sides start from identical bf16 values.

Every tensor is drawn from its own torch.Generator seeded from
(workload seed, tensor name[, index]), so a tensor can be regenerated alone
(e.g. one chunk of a 32k-token prefix) without drawing the others.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

BLOCK = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    """Drafter shape plus the per-step workload around it."""

    name: str
    num_layers: int
    hidden: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    num_target_layers: int
    target_hidden: int
    dtype: str  # "f32" or "bf16"
    batch: int
    ctx_min: int  # context length after this step's injection, inclusive range
    ctx_max: int
    num_passes: int = 1
    commit_per_pass: int = 0
    match_prob: Sequence[float] = (0.8,)  # per drafted position (len 1 = constant)
    block_size: int = BLOCK
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    new_rows: int = BLOCK  # context rows injected per sequence per step
    seed: int = 0
    # "dtype": projection matrices in the drafter dtype; "fp8": FP8 E4M3
    # codes with one float32 scale per output row (bf16 drafters)
    weight_format: str = "dtype"

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    @property
    def rows(self) -> int:
        return self.batch * self.block_size

    @property
    def drafts_per_step(self) -> int:
        return self.batch * (self.block_size - 1)

    def match_probs(self) -> np.ndarray:
        """Match probability for drafted positions 1..K-1 (length K-1)."""
        p = np.asarray(self.match_prob, dtype=np.float64)
        if p.size == 1:
            p = np.full(self.block_size - 1, float(p[0]))
        assert p.size == self.block_size - 1
        return p

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _decay_schedule(p_first: float, p_last: float, k: int) -> tuple:
    # Linear in the block index j = 1..k with p(1) = p_first and p(k) = p_last;
    # slot k is the bonus slot and is never compared, so only 1..k-1 are kept.
    step = (p_first - p_last) / (k - 1)
    return tuple(p_first - step * (j - 1) for j in range(1, k))


_QWEN = dict(hidden=4096, num_q_heads=32, num_kv_heads=8, head_dim=128,
             intermediate=12288, vocab=151936, num_target_layers=5,
             target_hidden=4096, dtype="bf16")

WORKLOADS: Dict[str, Workload] = {
    "tiny-f32": Workload(
        name="tiny-f32", num_layers=1, hidden=256, num_q_heads=4,
        num_kv_heads=2, head_dim=64, intermediate=768, vocab=1024,
        num_target_layers=3, target_hidden=256, dtype="f32", batch=1,
        ctx_min=128, ctx_max=128, match_prob=(0.8,), seed=1001),
    "qwen3-8b-1L-b1-ctx2048": Workload(
        name="qwen3-8b-1L-b1-ctx2048", num_layers=1, batch=1, ctx_min=2048,
        ctx_max=2048, match_prob=(0.8,), seed=1002, **_QWEN),
    "qwen3-8b-5L-b16-ctx1k-4k": Workload(
        name="qwen3-8b-5L-b16-ctx1k-4k", num_layers=5, batch=16,
        ctx_min=1024, ctx_max=4096, match_prob=(0.8,), seed=1003, **_QWEN),
    "qwen3-8b-3L-b4-ctx32k": Workload(
        name="qwen3-8b-3L-b4-ctx32k", num_layers=3, batch=4, ctx_min=32768,
        ctx_max=32768, match_prob=_decay_schedule(0.9, 0.3, BLOCK), seed=1004,
        **_QWEN),
    "qwen3-8b-3L-b64-ctx256-2k-S2": Workload(
        name="qwen3-8b-3L-b64-ctx256-2k-S2", num_layers=3, batch=64,
        ctx_min=256, ctx_max=2048, num_passes=2, commit_per_pass=8,
        match_prob=(0.75,), seed=1005, **_QWEN),
}
# Order of the five workloads: tiny parity case first, then the batch-1
# Qwen3-8B-shaped drafter, then the batched ones.
WORKLOAD_ORDER: List[str] = list(WORKLOADS)
# The batch-1 drafter with FP8 E4M3 projection weights (per-row scales).
WORKLOADS["qwen3-8b-1L-b1-ctx2048-fp8"] = WORKLOADS[
    "qwen3-8b-1L-b1-ctx2048"].replace(name="qwen3-8b-1L-b1-ctx2048-fp8",
                                      weight_format="fp8")
EXTRA_WORKLOADS: List[str] = ["qwen3-8b-1L-b1-ctx2048-fp8"]
HEADLINE = "qwen3-8b-1L-b1-ctx2048"
# The benchmark's headline line: the largest workload that fits one GPU
# (batch 64, two refinement passes); the others follow in the same line.
BENCH_DEFAULT = "qwen3-8b-3L-b64-ctx256-2k-S2"


def small_bf16(**kw) -> Workload:
    """A small bf16 drafter used by tests: several tiles, ragged tails."""
    base = dict(name="small-bf16", num_layers=2, hidden=512, num_q_heads=8,
                num_kv_heads=2, head_dim=64, intermediate=1408, vocab=4000,
                num_target_layers=3, target_hidden=384, dtype="bf16", batch=3,
                ctx_min=40, ctx_max=300, match_prob=(0.8,), seed=77)
    base.update(kw)
    return Workload(**base)


# --------------------------------------------------------------------------
# seeded generators
# --------------------------------------------------------------------------

def _seed(wl_seed: int, name: str, index: int = 0) -> int:
    h = hashlib.sha256(f"{wl_seed}/{name}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, wl_seed, name, index=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wl_seed, name, index))
    return g


def torch_dtype(wl: Workload) -> torch.dtype:
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def normal(wl: Workload, name: str, shape, std: float, device="cpu",
           index: int = 0) -> torch.Tensor:
    g = _gen(device, wl.seed, name, index)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch_dtype(wl))


def uniform_gains(wl: Workload, name: str, n: int, device="cpu") -> torch.Tensor:
    g = _gen(device, wl.seed, name)
    t = torch.rand(n, generator=g, device=device, dtype=torch.float32) + 0.5
    return t.to(torch_dtype(wl))


def gen_weights(wl: Workload, device="cpu", random_gains: bool = False,
                std: float = 0.02) -> Dict[str, object]:
    """All drafter weights, PyTorch Linear layout [out, in].

    Per-layer tensors are lists indexed by layer.  Norm gains are 1.0 unless
    ``random_gains`` draws them from U(0.5, 1.5) to exercise the gain path.
    """
    D, I, V = wl.hidden, wl.intermediate, wl.vocab
    qd = wl.num_q_heads * wl.head_dim
    kvd = wl.num_kv_heads * wl.head_dim
    dt = torch_dtype(wl)

    def gain(name):
        if random_gains:
            return uniform_gains(wl, name, D, device)
        return torch.ones(D, dtype=dt, device=device)

    w: Dict[str, object] = {
        "embed": normal(wl, "embed", (V, D), std, device),
        "fc": normal(wl, "fc", (D, wl.num_target_layers * wl.target_hidden),
                     std, device),
        "hidden_norm": gain("hidden_norm"),
        "final_norm": gain("final_norm"),
        "lm_head": normal(wl, "lm_head", (V, D), std, device),
    }
    for key in ("attn_norm", "mlp_norm"):
        w[key] = [gain(f"{key}{l}") for l in range(wl.num_layers)]
    shapes = {"wq": (qd, D), "wk": (kvd, D), "wv": (kvd, D), "wo": (D, qd),
              "w_gate": (I, D), "w_up": (I, D), "w_down": (D, I)}
    for key, shp in shapes.items():
        w[key] = [normal(wl, key, shp, std, device, index=l)
                  for l in range(wl.num_layers)]
    if wl.weight_format == "fp8":
        for key in ("fc", "lm_head"):
            w[key], w[key + "_scale"] = to_fp8_rows(w[key])
        for key in shapes:
            pairs = [to_fp8_rows(t) for t in w[key]]
            w[key] = [c for c, _ in pairs]
            w[key + "_scale"] = [sc for _, sc in pairs]
    return w


def to_fp8_rows(t: torch.Tensor):
    """FP8 E4M3 storage of a [out, in] matrix with one float32 scale per
    output row: scale = max |row| / 448 (the largest E4M3 value), codes =
    torch's own round-to-nearest conversion of row / scale (clamped to the
    E4M3 range).  Returns (codes as torch.float8_e4m3fn, scales)."""
    x = t.to(torch.float32)
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x / scale[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q, scale.contiguous()


def gen_hiddens(wl: Workload, rows: int, device="cpu", index: int = 0,
                tag: str = "hidden") -> List[torch.Tensor]:
    """n_t target hidden-state matrices [rows, D_t], N(0, 1), chunk ``index``."""
    return [normal(wl, f"{tag}{k}", (rows, wl.target_hidden), 1.0, device,
                   index=index) for k in range(wl.num_target_layers)]


def gen_ctx_lens(wl: Workload) -> np.ndarray:
    """Context length per sequence after this step's injection (inclusive)."""
    rng = np.random.default_rng(_seed(wl.seed, "ctx_len"))
    if wl.ctx_min == wl.ctx_max:
        return np.full(wl.batch, wl.ctx_max, dtype=np.int32)
    return rng.integers(wl.ctx_min, wl.ctx_max + 1, size=wl.batch,
                        dtype=np.int64).astype(np.int32)


def gen_anchors(wl: Workload, index: int = 0) -> np.ndarray:
    rng = np.random.default_rng(_seed(wl.seed, "anchor", index))
    return rng.integers(0, wl.vocab - 1, size=wl.batch,
                        dtype=np.int64).astype(np.int32)


def gen_verify_draws(wl: Workload, index: int = 0) -> Dict[str, np.ndarray]:
    """Random draws of the synthetic target for one step.

    u[b, j] ~ U[0, 1) decides whether drafted position j+1 matches;
    r[b, j] in [0, V-2] picks the mismatching token; tail[b] in [0, V-1] is
    the target's token at the bonus slot (block index K).
    """
    rng = np.random.default_rng(_seed(wl.seed, "verify", index))
    k1 = wl.block_size - 1
    u = rng.random((wl.batch, k1), dtype=np.float64).astype(np.float32)
    r = rng.integers(0, wl.vocab - 1, size=(wl.batch, k1),
                     dtype=np.int64).astype(np.int32)
    tail = rng.integers(0, wl.vocab, size=wl.batch,
                        dtype=np.int64).astype(np.int32)
    return {"u": u, "r": r, "tail": tail,
            "p": wl.match_probs().astype(np.float32)}


def gen_kv_prefix(wl: Workload, layer: int, kind: str, seq: int, length: int,
                  device="cpu", std: float = 1.28) -> torch.Tensor:
    """Directly seeded context K or V for one (layer, sequence): [Hkv, length, d].

    Used by full-size draft tests, where injecting the whole prefix through the
    oracle would take too long: the prefix then enters both sides as data.
    The default std matches what injection produces with N(0, 0.02) weights on
    unit-RMS features (0.02 * sqrt(4096) = 1.28).
    """
    name = f"kvprefix-{kind}"
    return normal(wl, name, (wl.num_kv_heads, length, wl.head_dim), std,
                  device, index=layer * 100003 + seq)


def to_f64(t) -> np.ndarray:
    """Exact host copy in float64 (bf16 and f32 values are exact in f64)."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def gen_target_weights(wl: Workload, device="cpu", std: float = 0.02,
                       head_std: float = 0.1):
    """Seeded weights of the small stand-in target model whose hooked layers
    feed the drafter: embedding [V, D_t], n_t residual layers [D_t, D_t]
    with RMSNorm gains U(0.5, 1.5), greedy head [V, D_t]; bf16 values.  The
    head's scale puts logits at a few units, as a trained head's are, so
    near ties between its top two tokens are rare."""
    Dt, V, nt = wl.target_hidden, wl.vocab, wl.num_target_layers
    bf = lambda t: t.to(torch.bfloat16)
    return {
        "embed": bf(normal(wl, "target-embed", (V, Dt), 1.0, device)
                    .float()),
        "layers": [bf(normal(wl, "target-layer", (Dt, Dt), std, device,
                             index=k).float()) for k in range(nt)],
        "gains": [bf(uniform_gains(wl, f"target-gain{k}", Dt, device)
                     .float()) for k in range(nt)],
        "head": bf(normal(wl, "target-head", (V, Dt), head_std, device)
                   .float()),
        "eps": wl.rms_eps,
    }


def gen_prompt(wl: Workload, length: int, index: int = 0) -> np.ndarray:
    """Seeded prompt token ids in [0, V - 2] (the mask id never occurs)."""
    rng = np.random.default_rng(_seed(wl.seed, "prompt", index))
    return rng.integers(0, wl.vocab - 1, size=length,
                        dtype=np.int64).astype(np.int32)
