"""C-ABI checks that need no GPU: the shared libraries load, export every
function that include/*.h declares (and nothing the binding expects is
missing), and host-side validation rejects bad calls before any launch.

No call here reaches a HIP runtime function: every case fails validation
first (the entry points validate all host arguments before launching)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import block_diffusion_drafting_dflash_amd as dfl
from block_diffusion_drafting_dflash_amd import binding
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = {"dflash.h": binding.LIB_PATH,
           "dflash_harness.h": binding.HARNESS_PATH}


@pytest.fixture(scope="module", autouse=True)
def built():
    if not (os.path.exists(binding.LIB_PATH) and
            os.path.exists(binding.HARNESS_PATH)):
        from block_diffusion_drafting_dflash_amd import build
        build.build()


def declared_functions(header: str):
    """Names of the functions a header declares inside its extern "C"
    block (comments stripped)."""
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(dflash_[a-z0-9_]+)\s*\(", text)))


def exported(lib_path: str):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path],
                         capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines()
            if len(line.split()) >= 3 and line.split()[1] == "T"}


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_every_declared_function_is_exported(header):
    names = declared_functions(header)
    assert names, f"no declarations parsed from {header}"
    syms = exported(HEADERS[header])
    missing = [n for n in names if n not in syms]
    assert not missing, f"{header}: not exported by the library: {missing}"
    lib = ctypes.CDLL(HEADERS[header])
    for n in names:
        assert getattr(lib, n) is not None


def test_binding_symbol_lists_match_headers():
    assert sorted(binding.LIB_SYMBOLS) == declared_functions("dflash.h")
    assert sorted(binding.HARNESS_SYMBOLS) == declared_functions(
        "dflash_harness.h")


def test_exports_are_only_the_declared_c_functions():
    """The library exports its C entry points unmangled; every exported
    dflash_* symbol is declared in the header."""
    syms = {s for s in exported(binding.LIB_PATH) if s.startswith("dflash_")}
    assert syms == set(declared_functions("dflash.h"))


def test_status_codes_match_header():
    text = open(os.path.join(ROOT, "include", "dflash.h")).read()
    codes = dict((n, int(v)) for n, v in
                 re.findall(r"(DFLASH_(?:OK|E_[A-Z]+))\s*=\s*(-?\d+)", text))
    assert {v: k for k, v in codes.items()} == binding.STATUS


# ---------------------------------------------------------------------------
# host-side validation (returns before any device work)

def lib():
    return binding.load_library()


def last_error():
    return lib().dflash_last_error().decode()


def good_config(**kw):
    wl = W.small_bf16()
    cfg = binding.make_config(wl)
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


@pytest.mark.parametrize("field,value,status,msg", [
    ("block_size", 8, "DFLASH_E_UNSUPPORTED", "block_size"),
    ("head_dim", 96, "DFLASH_E_UNSUPPORTED", "head_dim"),
    ("num_kv_heads", 3, "DFLASH_E_UNSUPPORTED", "num_kv_heads"),
    ("num_kv_heads", 8, "DFLASH_E_UNSUPPORTED", "num_kv_heads"),
    ("vocab", 4001, "DFLASH_E_UNSUPPORTED", "vocab"),
    ("hidden", 520, "DFLASH_E_UNSUPPORTED", "multiples of 64"),
    ("num_layers", 0, "DFLASH_E_INVALID", None),
    ("max_batch", 0, "DFLASH_E_INVALID", None),
    ("rope_theta", 0.0, "DFLASH_E_INVALID", "rope_theta"),
    ("num_target_layers", 9, "DFLASH_E_UNSUPPORTED", "num_target_layers"),
    ("mask_token_id", 4000, "DFLASH_E_INVALID", None),
    ("weight_format", 2, "DFLASH_E_INVALID", "weight_format"),
])
def test_create_rejects_bad_config(field, value, status, msg):
    cfg = good_config(**{field: value})
    out = ctypes.c_void_p()
    st = lib().dflash_create(ctypes.byref(cfg), None, ctypes.byref(out))
    assert binding.STATUS[st] == status, (st, last_error())
    assert out.value is None
    if msg:
        assert msg in last_error()


def _fake_weights(wl, scales):
    """Non-null, aligned stand-in pointers (never dereferenced: validation
    fails before any device work)."""
    n = wl.num_layers
    keep = []

    def lst(v):
        arr = (ctypes.c_void_p * n)(*([v] * n))
        keep.append(arr)
        return ctypes.cast(arr, binding._PP)

    w = binding.Weights(embed=4096, fc=4096, hidden_norm=4096,
                        final_norm=4096, lm_head=4096)
    for k in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate",
              "w_up", "w_down"):
        setattr(w, k, lst(4096))
    if scales:
        w.fc_scale = 4096
        w.lm_head_scale = 4096
        for k in binding.LAYER_MATRICES:
            setattr(w, k + "_scale", lst(4096))
    return w, keep


def test_create_rejects_fp8_without_scales_and_fp8_f32():
    wl = W.small_bf16(weight_format="fp8")
    cfg = binding.make_config(wl)
    assert cfg.weight_format == 1
    out = ctypes.c_void_p()
    w, keep = _fake_weights(wl, scales=False)
    st = lib().dflash_create(ctypes.byref(cfg), ctypes.byref(w),
                             ctypes.byref(out))
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    assert "FP8 weights" in last_error()
    w, keep2 = _fake_weights(wl, scales=True)
    w.wk_scale[1] = 4098  # misaligned scale vector of one layer
    st = lib().dflash_create(ctypes.byref(cfg), ctypes.byref(w),
                             ctypes.byref(out))
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    assert "wk_scale[1]" in last_error()
    f32 = binding.make_config(W.WORKLOADS["tiny-f32"].replace(
        weight_format="fp8"))
    st = lib().dflash_create(ctypes.byref(f32), ctypes.byref(w),
                             ctypes.byref(out))
    assert binding.STATUS[st] == "DFLASH_E_UNSUPPORTED"
    assert out.value is None


def test_create_rejects_null_weights_and_out():
    cfg = good_config()
    out = ctypes.c_void_p()
    st = lib().dflash_create(ctypes.byref(cfg), None, ctypes.byref(out))
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    assert "weights" in last_error()
    st = lib().dflash_create(ctypes.byref(cfg), None, None)
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    w = binding.Weights()
    st = lib().dflash_create(ctypes.byref(cfg), ctypes.byref(w),
                             ctypes.byref(out))
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    assert "NULL" in last_error()


def test_kv_cache_bytes_layout():
    wl = W.small_bf16()
    cfg = binding.make_config(wl, max_batch=5, max_ctx=1000)
    want = (wl.num_layers * 2 * 5 * wl.num_kv_heads * (1000 + 16) *
            wl.head_dim * 2)
    assert lib().dflash_kv_cache_bytes(ctypes.byref(cfg)) == want
    cfg.dtype = binding.DTYPE["f32"]
    assert lib().dflash_kv_cache_bytes(ctypes.byref(cfg)) == 2 * want
    cfg.max_batch = 0
    assert lib().dflash_kv_cache_bytes(ctypes.byref(cfg)) == 0


def test_kv_cache_paged_bytes_layout():
    wl = W.small_bf16()
    cfg = binding.make_config(wl, max_batch=5, max_ctx=1000)
    want = wl.num_layers * 2 * 37 * wl.num_kv_heads * 64 * wl.head_dim * 2
    assert lib().dflash_kv_cache_paged_bytes(ctypes.byref(cfg), 64, 37) == want
    assert binding.kv_cache_paged_bytes(cfg, 64, 37) == want
    assert lib().dflash_kv_cache_paged_bytes(ctypes.byref(cfg), 0, 37) == 0
    assert lib().dflash_kv_cache_paged_bytes(ctypes.byref(cfg), 64, 0) == 0
    assert lib().dflash_kv_cache_paged_bytes(None, 64, 37) == 0


def test_calls_with_null_context_are_rejected():
    L = lib()
    p = ctypes.c_void_p(16)
    st = L.dflash_inject_kv(None, None, None, 64, 1, p, p, p)
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    st = L.dflash_draft_block(None, None, 1, p, None, p, 10, p, 1, 0, p,
                              None, None, None)
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    st = L.dflash_draft_block_noalloc(None, None, 1, p, None, p, 10, p, 1, 0,
                                      p, None, None, None)
    assert binding.STATUS[st] == "DFLASH_E_INVALID"
    assert binding.STATUS[L.dflash_set_kernel_timing(None, 1)] == \
        "DFLASH_E_INVALID"
    assert binding.STATUS[L.dflash_check_device_errors(None, None, None)] == \
        "DFLASH_E_INVALID"
    assert binding.STATUS[L.dflash_set_kv_pages(None, 64, 4, p, 8)] == \
        "DFLASH_E_INVALID"


@pytest.mark.parametrize("batch,block,null,status", [
    (0, 16, False, "DFLASH_E_SHAPE"),
    (4, 0, False, "DFLASH_E_SHAPE"),
    (4, 65, False, "DFLASH_E_SHAPE"),
    (4, 16, True, "DFLASH_E_INVALID"),
])
def test_verify_validation(batch, block, null, status):
    p = ctypes.c_void_p(16)
    args = [None if null else p, p, p, p]
    st = lib().dflash_verify_greedy(None, batch, block, *args)
    assert binding.STATUS[st] == status


def test_harness_validation():
    h = binding.load_harness()
    p = ctypes.c_void_p(16)
    st = h.dflash_harness_synth_target(None, 0, 16, 100, p, p, p, p, p, p)
    assert st != 0
    st = h.dflash_harness_synth_target(None, 2, 16, 100, None, p, p, p, p, p)
    assert st != 0


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and fails loudly without its
    library."""
    pkg = os.path.dirname(dfl.__file__)
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", src, re.M), f
    assert "raise RuntimeError" in open(binding.__file__).read()


@pytest.mark.parametrize("batch,block,vocab,null,status", [
    (0, 16, 100, False, "DFLASH_E_SHAPE"),
    (4, 1, 100, False, "DFLASH_E_SHAPE"),
    (4, 65, 100, False, "DFLASH_E_SHAPE"),
    (4, 16, 0, False, "DFLASH_E_SHAPE"),
    (4, 16, 262145, False, "DFLASH_E_SHAPE"),
    (4, 16, 100, True, "DFLASH_E_INVALID"),
])
def test_verify_sampling_validation(batch, block, vocab, null, status):
    p = ctypes.c_void_p(16)
    args = [None if null else p] + [p] * 6
    st = lib().dflash_verify_sampling(None, batch, block, vocab, *args)
    assert binding.STATUS[st] == status


def test_bench_profile_bookkeeping():
    """The bench keys each committed HBM-traffic summary to the sources of
    its kernel class: every named source exists, and every summary under
    profiles/ names a known kernel class and workload and a well-formed
    hash and byte count (whether it still matches is decided at run time)."""
    import bench
    import workloads as W
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "block_diffusion_drafting_dflash_amd", "csrc")
    for kind, files in bench.KERNEL_SOURCES.items():
        for f in files + ["common.h", "kernels.h"]:
            assert os.path.exists(os.path.join(csrc, f)), (kind, f)
        assert re.fullmatch(r"[0-9a-f]{64}", bench.kernel_source_sha(kind))
    prof = os.path.join(root, "profiles")
    for f in os.listdir(prof):
        if not f.endswith("_traffic.txt"):
            continue
        kv = {}
        for line in open(os.path.join(prof, f)):
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        assert kv["kernel"] in bench.KERNEL_SOURCES, f
        assert kv["workload"] in W.WORKLOADS, f
        assert f == f"{kv['kernel']}_{kv['workload']}_traffic.txt"
        assert re.fullmatch(r"[0-9a-f]{64}", kv["source_sha256"]), f
        assert int(kv["traffic_bytes_per_launch"]) > 0, f
