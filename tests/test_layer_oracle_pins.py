"""Pins of the layer oracle (oracle/layer_ref.py) against things other than itself.

The linears, RMSNorm, SwiGLU and softmax against torch's own routines; the
rounding points against torch's bf16 cast; closed forms (zero weights, a
constant row, an identity lm-head); the composition against a torch chain;
and the cut against the uncut sampler (every operator after the layers acts
on one row at a time).  No GPU is used.
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import layer_ref as L
from oracle.fp8_ref import round_bf16


def _rng(*s):
    return np.random.default_rng([25, *s])


def _bf(x):
    return round_bf16(np.asarray(x, np.float64))


def _tbf(x):
    """torch's own bf16 rounding of fp32 values (fp64 -> fp32 is exact for the values used)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _layer(r, T=5, D=64, Hd=48, Fh=96):
    h = _bf(r.standard_normal((T, D)))
    o = _bf(0.5 * r.standard_normal((T, Hd)))
    w_o = _bf(0.1 * r.standard_normal((D, Hd)))
    g = _bf(1 + 0.1 * r.standard_normal(D))
    wg, wu = _bf(0.1 * r.standard_normal((Fh, D))), _bf(0.1 * r.standard_normal((Fh, D)))
    wd = _bf(0.1 * r.standard_normal((D, Fh)))
    return h, o, w_o, g, wg, wu, wd


def test_linear_and_rms_norm_match_torch():
    r = _rng(1)
    x, w = _bf(r.standard_normal((7, 40))), _bf(r.standard_normal((9, 40)))
    np.testing.assert_allclose(L.linear(x, w), F.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy(),
                               rtol=1e-13, atol=1e-13)
    g = _bf(1 + 0.1 * r.standard_normal(40))
    ref = F.rms_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(L.rms_norm_rows(x, g, 1e-5), ref, rtol=1e-13, atol=1e-13)
    # a constant row c: gamma c / sqrt(c^2 + eps)
    c = np.full((1, 40), 3.0)
    np.testing.assert_allclose(L.rms_norm_rows(c, g, 1e-5)[0], g * 3.0 / np.sqrt(9.0 + 1e-5), rtol=1e-14)


def test_rounding_points_match_torch_bf16_chain():
    # The same chain with torch's linear / rms_norm / silu and torch's bf16 cast
    # at each operator output (every pre-rounding value here is exact in fp32:
    # few terms of short bf16 products).
    r = _rng(2)
    T, D, Hd, Fh = 4, 8, 8, 16
    q = lambda s: _bf(np.round(r.standard_normal(s) * 4) / 4)        # quarter steps: short products
    h, o, w_o = q((T, D)), q((T, Hd)), q((D, Hd))
    g = np.ones(D)
    wg, wu, wd = q((Fh, D)), q((Fh, D)), q((D, Fh))
    got = L.layer0_finish(h, o, w_o, g, wg, wu, wd, 1e-5)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    a = _tbf(F.linear(t(o), t(w_o)).numpy())
    rr = _tbf(t(h).numpy() + a)
    x = _tbf(F.rms_norm(t(rr), (D,), t(g), eps=1e-5).numpy())
    gate, up = _tbf(F.linear(t(x), t(wg)).numpy()), _tbf(F.linear(t(x), t(wu)).numpy())
    y = _tbf((F.silu(t(gate)) * t(up)).numpy())
    d = _tbf(F.linear(t(y), t(wd)).numpy())
    out = _tbf(rr + d)
    for k, v in dict(a=a, r=rr, gate=gate, up=up, y=y, d=d, out=out).items():
        np.testing.assert_array_equal(got[k], v, err_msg=k)
    # x: torch's fp64 rms_norm cast to bf16 via fp32 (double rounding is possible
    # in principle; none of these values sits that close to a tie)
    np.testing.assert_array_equal(got["x"], x)


def test_closed_forms_of_the_layer():
    r = _rng(3)
    h, o, w_o, g, wg, wu, wd = _layer(r)
    z = L.layer0_finish(h, o, np.zeros_like(w_o), g, wg, wu, wd, 1e-5)
    np.testing.assert_array_equal(z["r"], h)                          # no attention contribution
    z = L.layer0_finish(h, o, w_o, g, wg, wu, np.zeros_like(wd), 1e-5)
    np.testing.assert_array_equal(z["out"], z["r"])                   # no FFN contribution
    z = L.layer0_finish(h, o, w_o, g, np.zeros_like(wg), wu, wd, 1e-5)
    np.testing.assert_array_equal(z["y"], 0 * z["y"])                 # silu(0) = 0
    z = L.layer0_finish(np.zeros_like(h), o, w_o, g, wg, wu, wd, 1e-5)
    np.testing.assert_array_equal(z["r"], z["a"])                     # r = a exactly when h = 0


def test_residual_adds_the_rounded_projection():
    # random bf16 operands: a = bf16(torch's O W_o^T) is not exact in bf16,
    # and r = bf16(h + a) (both roundings by the pinned bf16 rounding)
    r = _rng(8)
    h, o, w_o, g, wg, wu, wd = _layer(r)
    got = L.layer0_finish(h, o, w_o, g, wg, wu, wd, 1e-5)
    a = round_bf16(F.linear(torch.from_numpy(o), torch.from_numpy(w_o)).numpy())
    np.testing.assert_array_equal(got["a"], a)
    np.testing.assert_array_equal(got["r"], round_bf16(h + a))
    x = round_bf16(F.rms_norm(torch.from_numpy(got["r"]), (h.shape[1],), torch.from_numpy(g), eps=1e-5).numpy())
    np.testing.assert_array_equal(got["x"], x)


def test_gate_and_up_are_not_interchangeable():
    r = _rng(4)
    h, o, w_o, g, wg, wu, wd = _layer(r)
    a = L.layer0_finish(h, o, w_o, g, wg, wu, wd, 1e-5)
    b = L.layer0_finish(h, o, w_o, g, wu, wg, wd, 1e-5)
    assert np.max(np.abs(a["y"] - b["y"])) > 1e-2


def test_softmax_argmax_against_torch():
    r = _rng(5)
    logits = r.standard_normal((6, 300)) * 5
    logits[2, 17] = logits[2, 40] = logits[2].max() + 1.0              # a tie: the first index wins
    p = L.softmax_rows(logits)
    np.testing.assert_allclose(p, torch.softmax(torch.from_numpy(logits), -1).numpy(), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    out = L.sample_rows(np.eye(6, 8), np.ones(8), np.ones((300, 8)), 1e-5)   # all logits equal: token 0
    assert np.all(out["token"] == 0)
    tok = np.argmax(logits, -1)                      # the oracle's decision rule
    assert tok[2] == 17
    np.testing.assert_array_equal(tok, torch.argmax(torch.from_numpy(logits), -1).numpy())


def test_identity_lm_head_closed_form():
    # W_lm = c I (V = D): logits = c z, the token is argmax z, the confidence
    # 1 / sum exp(c (z - max z)).
    r = _rng(6)
    D = 32
    hid = _bf(r.standard_normal((3, D)))
    g = np.ones(D)
    out = L.sample_rows(hid, g, 2.0 * np.eye(D), 1e-5)
    z = L.final_norm(hid, g, 1e-5)
    np.testing.assert_array_equal(out["logits"], (2.0 * z).astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(out["token"], np.argmax(z, -1))
    np.testing.assert_allclose(out["confidence"], 1.0 / np.exp(2.0 * (z - z.max(-1, keepdims=True))).sum(-1),
                               rtol=1e-13)
    # with a non-unit gamma: z is torch's rms_norm rounded to bf16
    g = _bf(1 + 0.2 * r.standard_normal(D))
    out = L.sample_rows(hid, g, np.eye(D), 1e-5)
    zt = F.rms_norm(torch.from_numpy(hid), (D,), torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_array_equal(out["z"], round_bf16(zt))


def test_the_cut_equals_the_uncut_sampler_on_block_rows():
    r = _rng(7)
    D, V = 48, 200
    seqs = [(0, 30, 8, 16), (30, 20, 0, 4), (50, 25, 17, 25)]     # (offset, len, block_start, block_end)
    hid = _bf(r.standard_normal((75, D)))
    g = _bf(1 + 0.1 * r.standard_normal(D))
    w = _bf(0.2 * r.standard_normal((V, D)))
    cut = L.sampler_cut(hid, seqs, g, w, 1e-5)
    full = L.sampler_all_rows(hid, g, w, 1e-5)
    rows = np.r_[8:16, 30:34, 67:75]
    np.testing.assert_array_equal(cut["rows"], rows)
    for k in ("logits", "probs", "token", "confidence"):
        np.testing.assert_array_equal(cut[k], full[k][rows], err_msg=k)
    # another sample order permutes the outputs the same way
    perm = L.sampler_cut(hid, [seqs[2], seqs[0], seqs[1]], g, w, 1e-5)
    np.testing.assert_array_equal(perm["token"], np.r_[cut["token"][12:], cut["token"][:12]])
