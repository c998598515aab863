"""FP8 E4M3 weights with per-output-row scales: the oracle's decoding and
dequantisation, and the drafter with FP8 projections.  CPU only."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import OracleModel, draft_batch, inject_rows
from oracle.numerics import decode_e4m3, dequant_rows
from tests import floor_eval


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256)
    ours = decode_e4m3(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(
        torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    # signs of the two zeros
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xFE, -448.0),
    (0xB8, -1.0)])
def test_decode_closed_forms(code, value):
    assert decode_e4m3(np.array([code]))[0] == value


def test_decode_nan_codes():
    v = decode_e4m3(np.arange(256))
    assert set(np.nonzero(np.isnan(v))[0].tolist()) == {0x7F, 0xFF}
    # every finite value is an integer multiple of 2^-9 and distinct per sign
    fin = v[~np.isnan(v)]
    assert np.all(np.round(fin * 512) == fin * 512)
    assert len(set(np.abs(fin).tolist())) == 127


def test_row_quantisation_of_the_generator_is_within_half_an_ulp():
    wl = W.small_bf16(weight_format="fp8")
    t = W.normal(wl, "q", (64, 256), 0.02)
    q, sc = W.to_fp8_rows(t)
    w = t.double().numpy()
    deq = dequant_rows(q.view(torch.uint8).numpy(), sc.double().numpy())
    # scale: the row's largest magnitude maps to 448
    np.testing.assert_allclose(np.abs(w).max(1), 448 * sc.double().numpy(),
                               rtol=1e-7)
    # relative spacing of E4M3 normals is 2^-3: error <= half of it (or half
    # the subnormal spacing 2^-9 in units of the scale)
    err = np.abs(deq - w)
    half = np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * sc.double().numpy()
                      [:, None])
    assert np.all(err <= half * (1 + 1e-9))


def _fp8_and_plain(wl):
    """FP8 weights, and the same weights dequantised into plain float64
    arrays (what the FP8 drafter must compute with)."""
    w = W.gen_weights(wl, random_gains=True)
    plain = {}
    for k, v in w.items():
        if k.endswith("_scale"):
            continue
        sc = w.get(k + "_scale")
        if sc is None:
            plain[k] = v
        elif isinstance(v, list):
            plain[k] = [dequant_rows(c.view(torch.uint8).numpy(),
                                     s.double().numpy()) for c, s in zip(v, sc)]
        else:
            plain[k] = dequant_rows(v.view(torch.uint8).numpy(),
                                    sc.double().numpy())
    return w, plain


def test_fp8_drafter_is_the_drafter_of_the_dequantised_weights():
    wl = W.small_bf16(weight_format="fp8", batch=1, ctx_min=40, ctx_max=40)
    w, plain = _fp8_and_plain(wl)
    H = W.gen_hiddens(wl, 40)
    pos = np.arange(40)
    m8, mp = OracleModel(wl, w), OracleModel(wl, plain)
    mp.W_lm = plain["lm_head"]  # float64 (a plain model keeps float32)
    c8, cp = inject_rows(m8, H, pos), inject_rows(mp, H, pos)
    for l in c8:
        np.testing.assert_array_equal(c8[l][0], cp[l][0])
        np.testing.assert_array_equal(c8[l][1], cp[l][1])
    r8 = draft_batch(m8, [c8], [40], anchors=[7], keep_logits=True)[0]
    rp = draft_batch(mp, [cp], [40], anchors=[7], keep_logits=True)[0]
    np.testing.assert_allclose(r8["logits"][0], rp["logits"][0], rtol=0,
                               atol=1e-12)


def test_fp8_rounding_points_match_torch_composition():
    """The float64 torch composition (codes widened, scale after the
    product) reproduces the FP8 oracle: injection and a pass."""
    wl = W.small_bf16(weight_format="fp8", batch=1, ctx_min=60, ctx_max=60,
                      seed=92)
    w = W.gen_weights(wl, random_gains=True)
    H = W.gen_hiddens(wl, 60)
    pos = np.arange(60)
    model = OracleModel(wl, w)
    ctx = inject_rows(model, H, pos)
    ref = draft_batch(model, [ctx], [60], anchors=[11], keep_logits=True)[0]
    p = floor_eval.Prepared(wl, w, torch.float64)
    inj = floor_eval.inject(p, H, pos)
    for l in ctx:
        np.testing.assert_allclose(inj[l][0], ctx[l][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(inj[l][1], ctx[l][1], rtol=0, atol=1e-12)
    blk = np.full(16, wl.mask_id)
    blk[0] = 11
    _, z = floor_eval.pass_logits(p, inj, 60, blk)
    np.testing.assert_allclose(z, ref["logits"][0], rtol=0, atol=1e-12)
