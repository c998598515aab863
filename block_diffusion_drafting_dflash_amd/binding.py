"""ctypes binding for libdflash.so (argument marshalling only).

Every computation of the drafting step runs in the HIP library; this module
turns torch tensors into device pointers, keeps the weight tensors alive for
the context's lifetime and raises on non-OK statuses.  If the library has
not been built, loading fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB may name another build of the same library (the host-sanitized
# one that the ABI tests load); by default the in-tree build
LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(_HERE, "libdflash.so")
HARNESS_PATH = os.path.join(_HERE, "libdflash_harness.so")

DFLASH_OK = 0
STATUS = {0: "DFLASH_OK", -1: "DFLASH_E_INVALID", -2: "DFLASH_E_SHAPE",
          -3: "DFLASH_E_CAPACITY", -4: "DFLASH_E_DEVICE",
          -5: "DFLASH_E_UNSUPPORTED"}
DTYPE = {"f32": 0, "bf16": 1}
WEIGHT_FORMAT = {"dtype": 0, "fp8": 1}

# C-ABI symbols declared in include/dflash.h and include/dflash_harness.h
LIB_SYMBOLS = ["dflash_create", "dflash_destroy", "dflash_kv_cache_bytes",
               "dflash_last_error", "dflash_check_device_errors",
               "dflash_inject_kv", "dflash_draft_block",
               "dflash_verify_greedy", "dflash_verify_sampling",
               "dflash_set_kernel_timing", "dflash_get_kernel_timing",
               "dflash_set_kv_pages", "dflash_kv_cache_paged_bytes",
               "dflash_draft_block_noalloc"]
TIME_KIND = {"off": 0, "lmhead": 1, "attention": 2, "gemm": 3}
HARNESS_SYMBOLS = ["dflash_harness_synth_target",
                   "dflash_harness_fp8_to_bf16",
                   "dflash_harness_target_forward",
                   "dflash_harness_read_probe"]


class DFlashError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "hidden", "num_q_heads", "num_kv_heads", "head_dim",
        "intermediate", "vocab", "num_target_layers", "target_hidden",
        "block_size", "mask_token_id", "dtype", "max_batch", "max_ctx",
        "max_inject_rows")] + [("rope_theta", ctypes.c_float),
                               ("rms_eps", ctypes.c_float),
                               ("weight_format", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)

LAYER_MATRICES = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("fc", ctypes.c_void_p),
                ("hidden_norm", ctypes.c_void_p)] + [
        (n, _PP) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                           "w_gate", "w_up", "w_down")] + [
        ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
        ("fc_scale", ctypes.c_void_p)] + [
        (n + "_scale", _PP) for n in LAYER_MATRICES] + [
        ("lm_head_scale", ctypes.c_void_p)]


_lib = None
_harness = None


def load_library():
    """Load libdflash.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} not found: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.dflash_create.argtypes = [ctypes.POINTER(Config),
                                  ctypes.POINTER(Weights),
                                  ctypes.POINTER(vp)]
    lib.dflash_create.restype = ctypes.c_int
    lib.dflash_destroy.argtypes = [vp]
    lib.dflash_destroy.restype = None
    lib.dflash_kv_cache_bytes.argtypes = [ctypes.POINTER(Config)]
    lib.dflash_kv_cache_bytes.restype = ctypes.c_size_t
    lib.dflash_last_error.argtypes = []
    lib.dflash_last_error.restype = ctypes.c_char_p
    lib.dflash_check_device_errors.argtypes = [vp, vp,
                                               ctypes.POINTER(i32)]
    lib.dflash_check_device_errors.restype = ctypes.c_int
    lib.dflash_inject_kv.argtypes = [vp, vp, _PP, i64, i32, vp, vp, vp]
    lib.dflash_inject_kv.restype = ctypes.c_int
    lib.dflash_draft_block.argtypes = [vp, vp, i32, vp, vp, vp, i32, vp, i32,
                                       i32, vp, vp, vp, vp]
    lib.dflash_draft_block.restype = ctypes.c_int
    lib.dflash_draft_block_noalloc.argtypes = lib.dflash_draft_block.argtypes
    lib.dflash_draft_block_noalloc.restype = ctypes.c_int
    lib.dflash_verify_greedy.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.dflash_verify_greedy.restype = ctypes.c_int
    lib.dflash_verify_sampling.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp,
                                           vp, vp, vp]
    lib.dflash_verify_sampling.restype = ctypes.c_int
    lib.dflash_set_kernel_timing.argtypes = [vp, i32]
    lib.dflash_set_kernel_timing.restype = ctypes.c_int
    lib.dflash_get_kernel_timing.argtypes = [vp, ctypes.POINTER(i32),
                                             ctypes.POINTER(ctypes.c_double)]
    lib.dflash_get_kernel_timing.restype = ctypes.c_int
    lib.dflash_set_kv_pages.argtypes = [vp, i32, i32, vp, i32]
    lib.dflash_set_kv_pages.restype = ctypes.c_int
    lib.dflash_kv_cache_paged_bytes.argtypes = [ctypes.POINTER(Config), i32,
                                                i32]
    lib.dflash_kv_cache_paged_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def load_harness():
    global _harness
    if _harness is not None:
        return _harness
    if not os.path.exists(HARNESS_PATH):
        raise RuntimeError(f"{HARNESS_PATH} not found: build it first")
    h = ctypes.CDLL(HARNESS_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    h.dflash_harness_synth_target.argtypes = [vp, i32, i32, i32, vp, vp, vp,
                                              vp, vp, vp]
    h.dflash_harness_synth_target.restype = ctypes.c_int
    h.dflash_harness_fp8_to_bf16.argtypes = [vp, i32, vp, vp]
    h.dflash_harness_fp8_to_bf16.restype = ctypes.c_int
    h.dflash_harness_target_forward.argtypes = [
        vp, i32, i32, i32, i32, vp, vp, _PP, _PP, vp, ctypes.c_float, _PP,
        ctypes.c_int64, vp, vp]
    h.dflash_harness_target_forward.restype = ctypes.c_int
    h.dflash_harness_read_probe.argtypes = [vp, vp, ctypes.c_int64, i32, vp]
    h.dflash_harness_read_probe.restype = ctypes.c_int
    _harness = h
    return h


def _check(status: int):
    if status != DFLASH_OK:
        msg = load_library().dflash_last_error().decode(errors="replace")
        raise DFlashError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(wl, max_batch=None, max_ctx=None,
                max_inject_rows=None) -> Config:
    """dflash_config for a workloads.Workload."""
    return Config(
        num_layers=wl.num_layers, hidden=wl.hidden,
        num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
        head_dim=wl.head_dim, intermediate=wl.intermediate, vocab=wl.vocab,
        num_target_layers=wl.num_target_layers,
        target_hidden=wl.target_hidden, block_size=wl.block_size,
        mask_token_id=wl.mask_id, dtype=DTYPE[wl.dtype],
        max_batch=max_batch or wl.batch, max_ctx=max_ctx or wl.ctx_max,
        max_inject_rows=max_inject_rows or max(wl.batch * wl.new_rows, 2048),
        rope_theta=wl.rope_theta, rms_eps=wl.rms_eps,
        weight_format=WEIGHT_FORMAT[getattr(wl, "weight_format", "dtype")])


def kv_cache_bytes(cfg: Config) -> int:
    return int(load_library().dflash_kv_cache_bytes(ctypes.byref(cfg)))


def kv_cache_paged_bytes(cfg: Config, page_size: int, num_pages: int) -> int:
    return int(load_library().dflash_kv_cache_paged_bytes(
        ctypes.byref(cfg), page_size, num_pages))


class DFlash:
    """A drafting context on the current device (one per drafter)."""

    def __init__(self, wl, weights: Dict[str, object], max_batch=None,
                 max_ctx=None, max_inject_rows=None):
        self.lib = load_library()
        self.wl = wl
        self.cfg = make_config(wl, max_batch, max_ctx, max_inject_rows)
        self.weights = weights  # keep tensors alive
        self._arrays = []
        n = wl.num_layers

        def plist(key):
            arr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in weights[key]])
            self._arrays.append(arr)
            return ctypes.cast(arr, _PP)

        w = Weights(embed=weights["embed"].data_ptr(),
                    fc=weights["fc"].data_ptr(),
                    hidden_norm=weights["hidden_norm"].data_ptr(),
                    final_norm=weights["final_norm"].data_ptr(),
                    lm_head=weights["lm_head"].data_ptr())
        for key in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
                    "w_up", "w_down"):
            setattr(w, key, plist(key))
        if weights.get("fc_scale") is not None:  # FP8 E4M3 projections
            w.fc_scale = weights["fc_scale"].data_ptr()
            w.lm_head_scale = weights["lm_head_scale"].data_ptr()
            for key in LAYER_MATRICES:
                setattr(w, key + "_scale", plist(key + "_scale"))
        self._w = w
        ctx = ctypes.c_void_p()
        _check(self.lib.dflash_create(ctypes.byref(self.cfg), ctypes.byref(w),
                                      ctypes.byref(ctx)))
        self.ctx = ctx

    def close(self):
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            self.lib.dflash_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- tensors ------------------------------------------------------------
    @property
    def torch_dtype(self):
        return torch.float32 if self.wl.dtype == "f32" else torch.bfloat16

    def kv_cache_bytes(self) -> int:
        return kv_cache_bytes(self.cfg)

    def new_kv_cache(self, device="cuda") -> torch.Tensor:
        """[N_l, 2, max_batch, Hkv, max_ctx + K, d] in the drafter dtype."""
        c = self.cfg
        return torch.zeros(c.num_layers, 2, c.max_batch, c.num_kv_heads,
                           c.max_ctx + c.block_size, c.head_dim,
                           dtype=self.torch_dtype, device=device)

    def set_kv_pages(self, page_size: int, num_pages: int = 0,
                     block_table: Optional[torch.Tensor] = None):
        """Paged cache addressing for the following calls (page_size 0:
        contiguous).  block_table: [max_batch, pages per slot] int32 on the
        device, kept alive by this object while in use."""
        if page_size == 0:
            _check(self.lib.dflash_set_kv_pages(self.ctx, 0, 0, None, 0))
            self._block_table = None
            return
        if (block_table.dtype != torch.int32 or block_table.dim() != 2
                or not block_table.is_contiguous()):
            raise ValueError("block_table: contiguous int32 [max_batch, ld]")
        _check(self.lib.dflash_set_kv_pages(
            self.ctx, page_size, num_pages, _ptr(block_table),
            block_table.shape[1]))
        self._block_table = block_table

    def new_kv_cache_paged(self, page_size: int, num_pages: int,
                           device="cuda") -> torch.Tensor:
        """[N_l, 2, num_pages, Hkv, page_size, d] in the drafter dtype."""
        c = self.cfg
        return torch.zeros(c.num_layers, 2, num_pages, c.num_kv_heads,
                           page_size, c.head_dim, dtype=self.torch_dtype,
                           device=device)

    # -- entry points -------------------------------------------------------
    def inject_kv(self, hiddens: Sequence[torch.Tensor], row_seq: torch.Tensor,
                  row_pos: torch.Tensor, kv: torch.Tensor, stream=None):
        T = hiddens[0].shape[0]
        ld = hiddens[0].stride(0)
        arr = (ctypes.c_void_p * len(hiddens))(*[h.data_ptr() for h in hiddens])
        _check(self.lib.dflash_inject_kv(
            self.ctx, _stream(stream), ctypes.cast(arr, _PP), ld, T,
            _ptr(row_seq), _ptr(row_pos), _ptr(kv)))

    def draft_block(self, ctx_len: torch.Tensor, kv: torch.Tensor,
                    max_ctx_len: int, anchor: Optional[torch.Tensor] = None,
                    block_tokens: Optional[torch.Tensor] = None,
                    num_passes: int = 1, commit_per_pass: int = 0,
                    draft: Optional[torch.Tensor] = None,
                    conf: Optional[torch.Tensor] = None,
                    margin: Optional[torch.Tensor] = None,
                    logits: Optional[torch.Tensor] = None, stream=None,
                    noalloc: bool = False):
        """dflash_draft_block, or dflash_draft_block_noalloc (scratch in
        the library's static device buffer) with noalloc=True."""
        B = ctx_len.shape[0]
        K = self.cfg.block_size
        dev = ctx_len.device
        if draft is None:
            draft = torch.empty(B, K - 1, dtype=torch.int32, device=dev)
        fn = (self.lib.dflash_draft_block_noalloc if noalloc
              else self.lib.dflash_draft_block)
        _check(fn(
            self.ctx, _stream(stream), B, _ptr(anchor), _ptr(block_tokens),
            _ptr(ctx_len), int(max_ctx_len), _ptr(kv), num_passes,
            commit_per_pass, _ptr(draft), _ptr(conf), _ptr(margin),
            _ptr(logits)))
        return draft

    def set_kernel_timing(self, kind: str):
        _check(self.lib.dflash_set_kernel_timing(self.ctx, TIME_KIND[kind]))

    def kernel_timing(self):
        """(launches recorded, summed milliseconds) since the last call."""
        n = ctypes.c_int32(0)
        ms = ctypes.c_double(0.0)
        _check(self.lib.dflash_get_kernel_timing(self.ctx, ctypes.byref(n),
                                                 ctypes.byref(ms)))
        return n.value, ms.value

    def check_device_errors(self, stream=None) -> int:
        bits = ctypes.c_int32(0)
        st = self.lib.dflash_check_device_errors(self.ctx, _stream(stream),
                                                 ctypes.byref(bits))
        if st not in (DFLASH_OK, -4):
            _check(st)
        return bits.value


def verify_sampling(draft: torch.Tensor, draft_probs: torch.Tensor,
                    target_probs: torch.Tensor, u_accept: torch.Tensor,
                    u_sample: torch.Tensor,
                    accept: Optional[torch.Tensor] = None,
                    next_token: Optional[torch.Tensor] = None, stream=None):
    """Speculative-sampling verification (dflash_verify_sampling): draft
    [B, K-1] int32, draft_probs [B, K-1, V] and target_probs [B, K, V] fp32,
    u_accept [B, K-1] and u_sample [B] fp32, all contiguous on the device."""
    lib = load_library()
    B, K, V = target_probs.shape
    for t in (draft, draft_probs, target_probs, u_accept, u_sample):
        if not t.is_contiguous():
            raise ValueError("verify_sampling needs contiguous tensors")
    if accept is None:
        accept = torch.empty(B, dtype=torch.int32, device=target_probs.device)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32,
                                 device=target_probs.device)
    _check(lib.dflash_verify_sampling(_stream(stream), B, K, V, _ptr(draft),
                                      _ptr(draft_probs), _ptr(target_probs),
                                      _ptr(u_accept), _ptr(u_sample),
                                      _ptr(accept), _ptr(next_token)))
    return accept, next_token


def verify_greedy(draft: torch.Tensor, target: torch.Tensor,
                  accept: Optional[torch.Tensor] = None,
                  next_anchor: Optional[torch.Tensor] = None, stream=None):
    lib = load_library()
    B, K = target.shape
    if accept is None:
        accept = torch.empty(B, dtype=torch.int32, device=target.device)
    if next_anchor is None:
        next_anchor = torch.empty(B, dtype=torch.int32, device=target.device)
    _check(lib.dflash_verify_greedy(_stream(stream), B, K, _ptr(draft),
                                    _ptr(target), _ptr(accept),
                                    _ptr(next_anchor)))
    return accept, next_anchor


def fp8_to_bf16(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """The kernels' E4M3 -> bf16 widening of a uint8 code tensor (harness)."""
    h = load_harness()
    n = codes.numel()
    out = torch.empty(n, dtype=torch.int16, device=codes.device)
    st = h.dflash_harness_fp8_to_bf16(_stream(stream), n, _ptr(codes),
                                      _ptr(out))
    if st != 0:
        raise RuntimeError(f"dflash_harness_fp8_to_bf16 failed ({st})")
    return out


def read_probe(buf: torch.Tensor, grid: int, sink: torch.Tensor,
               stream=None) -> None:
    """The harness's plain streaming read of all of `buf` (a device tensor
    of a multiple of 256 KiB) by `grid` workgroups; `sink` an int32 device
    tensor it practically never writes."""
    h = load_harness()
    st = h.dflash_harness_read_probe(_stream(stream), _ptr(buf),
                                     buf.numel() * buf.element_size(),
                                     int(grid), _ptr(sink))
    if st != 0:
        raise RuntimeError(f"dflash_harness_read_probe failed ({st})")


def target_forward(tw, tokens: torch.Tensor, hooks=None, stream=None):
    """The harness's stand-in target over int32 `tokens` [rows]: returns
    (hooks: list of n_t bf16 [rows, D_t], next token [rows] int32, margin
    [rows] fp32).  tw: gen_target_weights' dict on the device."""
    h = load_harness()
    rows = tokens.numel()
    V, Dt = tw["embed"].shape
    nt = len(tw["layers"])
    dev = tokens.device
    if hooks is None:
        hooks = [torch.empty(rows, Dt, dtype=torch.bfloat16, device=dev)
                 for _ in range(nt)]
    nxt = torch.empty(rows, dtype=torch.int32, device=dev)
    margin = torch.empty(rows, dtype=torch.float32, device=dev)
    arr = lambda ts: ctypes.cast((ctypes.c_void_p * nt)(
        *[t.data_ptr() for t in ts]), _PP)
    st = h.dflash_harness_target_forward(
        _stream(stream), rows, nt, Dt, V, _ptr(tokens), _ptr(tw["embed"]),
        arr(tw["layers"]), arr(tw["gains"]), _ptr(tw["head"]),
        float(tw["eps"]), arr(hooks), hooks[0].stride(0), _ptr(nxt),
        _ptr(margin))
    if st != 0:
        raise RuntimeError(f"dflash_harness_target_forward failed ({st})")
    return hooks, nxt, margin


def synth_target(draft, u, r, tail, p, vocab, target=None, stream=None):
    h = load_harness()
    B, k1 = draft.shape
    if target is None:
        target = torch.empty(B, k1 + 1, dtype=torch.int32, device=draft.device)
    st = h.dflash_harness_synth_target(_stream(stream), B, k1 + 1, vocab,
                                       _ptr(draft), _ptr(u), _ptr(r),
                                       _ptr(tail), _ptr(p), _ptr(target))
    if st != 0:
        raise RuntimeError(f"dflash_harness_synth_target failed ({st})")
    return target
