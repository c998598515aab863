"""CPU oracle for the DFlash drafting step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy statement of what one drafting step computes:
feature fusion and KV injection, the single-pass (or S-pass) block draft, the
LM-head reduction, confidence-ordered commit, greedy verification and the
speculative-sampling verification for temperature > 0, plus the
accounting formulas the pages give (latency per token, the toy drafting race).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code, header, table or constant with it; both take their inputs
from the ``workloads`` generators only.

Sources (cited per function by page title and section):
  * "DFlash Guide: Block Diffusion for Speculative Decoding" (aifetchly blog)
  * "DFlash: Block Diffusion for Flash Speculative Decoding" (sciencestack
    abstract page, arXiv 2602.06036)
  * "DFlash: Diffusion Drafts the Block" (stable-lab tutorial chapter)

FP8 drafter weights (the guide's "FP4/FP8 mixed execution", section
"Production Benchmarks on NVIDIA Blackwell B200", names no format): a
projection may be given as FP8 E4M3 codes with one float32 scale per output
row; the oracle decodes the codes from the E4M3 definition and computes
with scale * value in float64, otherwise unchanged.

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except draft *quality* (acceptance on real text),
which needs trained weights: parity unpinned, and not claimed.
"""
from .numerics import (round_bf16, identity_round, rms_norm, silu, rope,
                       rope_angles, softmax, logsumexp, decode_e4m3,
                       dequant_rows)
from .drafter import (OracleModel, fuse_features, inject_kv, inject_rows,
                      block_attention, decoder_layer, lm_head_reduce,
                      confidence_commit, draft_sequence, draft_batch)
from .target import (TargetModel, target_forward, greedy_stream,
                     speculative_loop)
from .verify import (verify_greedy, verify_sampling, sample_inverse_cdf,
                     synthetic_target, expected_accept_len,
                     latency_per_token, simulate_rounds, toy_race_ratio,
                     simulate_toy_race)

__all__ = [
    "round_bf16", "identity_round", "rms_norm", "silu", "rope", "rope_angles",
    "softmax", "logsumexp", "OracleModel", "fuse_features", "inject_kv",
    "inject_rows", "block_attention", "decoder_layer", "lm_head_reduce",
    "confidence_commit", "draft_sequence", "draft_batch", "verify_greedy",
    "synthetic_target", "expected_accept_len", "latency_per_token",
    "simulate_rounds", "toy_race_ratio", "simulate_toy_race",
    "TargetModel", "target_forward", "greedy_stream", "speculative_loop",
]
