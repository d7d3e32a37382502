"""Pins of the multi-layer approximate-reuse oracle (oracle/multilayer_ref.py).

Closed cases of the schedule: with no edits since the refresh, or with a
single layer, or with a refresh at every step, the approximate step equals
the full recompute; with two layers and edits it does not (the stale keys are
really used).  The deeper layers' attention over mixed keys is checked
against torch's scaled_dot_product_attention, and the full forward's first
layer against the layer-0 oracle's full recompute.  No GPU is used.
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import lacache_ref as R
from oracle import multilayer_ref as ML
from oracle.fp8_ref import round_bf16
from exact_attention_state_amd import synth

D, H, DH, FF, V = 512, 4, 128, 256, 300


def _model(L, std=0.05):
    return synth.multilayer_params(D, H, DH, FF, L, V, qkv_std=std), R.Layer0Config(D, H, H, DH, 1e4, 1e-5)


def _steps(seqs, n, edits=3, seed=0):
    rng = np.random.default_rng([41, seed])
    T = max(o + l for o, l, _, _ in seqs)
    ids = [rng.integers(0, V, T)]
    for _ in range(n - 1):
        x = ids[-1].copy()
        for o, _, bs, be in seqs:
            x[o + bs + rng.integers(0, be - bs, edits)] = rng.integers(0, V, edits)
        ids.append(x)
    return ids


SEQS = [(0, 96, 64, 80), (96, 72, 16, 32)]


def test_no_edits_gives_the_full_recompute():
    p, cfg = _model(3)
    ids = _steps(SEQS, 1)
    out = ML.run_schedule(p, cfg, ids * 3, SEQS, None)
    assert out["refreshed"] == [True, False, False]
    for g, r in zip(out["got"], out["ref"]):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-9)


def test_one_layer_is_exact_under_edits():
    p, cfg = _model(1)
    out = ML.run_schedule(p, cfg, _steps(SEQS, 4), SEQS, None)
    for g, r in zip(out["got"], out["ref"]):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-9)


def test_refresh_every_step_is_exact_and_stale_keys_matter():
    p, cfg = _model(2)
    ids = _steps(SEQS, 4)
    out = ML.run_schedule(p, cfg, ids, SEQS, 1)
    assert all(out["refreshed"])
    for g, r in zip(out["got"], out["ref"]):
        np.testing.assert_array_equal(g, r)
    out = ML.run_schedule(p, cfg, ids, SEQS, None)
    err = [np.linalg.norm(g - r) / np.linalg.norm(r) for g, r in zip(out["got"], out["ref"])]
    assert err[0] == 0 and min(err[1:]) > 1e-4, err
    out2 = ML.run_schedule(p, cfg, ids, SEQS, 2)                      # a refresh at step 2 resets the error
    assert out2["refreshed"] == [True, False, True, False]
    np.testing.assert_array_equal(out2["got"][2], out2["ref"][2])


def test_first_layer_of_the_full_forward_is_the_layer0_recompute():
    p, cfg = _model(2)
    ids = _steps(SEQS, 1)[0]
    full = ML.forward_full(p, cfg, ids, SEQS)
    lp = p["layers"][0]
    params0 = {"embed": p["embed"], "gamma": lp["gamma_attn"], "w_qkv": lp["w_qkv"]}
    ref = R.full_recompute(params0, cfg, ids, SEQS)
    T = full["X"][0].shape[0]
    o = round_bf16(ref["out"].reshape(T, H * DH))
    from oracle.layer_ref import layer0_finish
    x1 = layer0_finish(full["X"][0], o, lp["w_o"], lp["gamma_ffn"], lp["w_gate"], lp["w_up"], lp["w_down"], 1e-5)
    np.testing.assert_allclose(full["X"][1], x1["out"], rtol=0, atol=0)


def test_deeper_attention_over_mixed_keys_matches_torch_sdpa():
    p, cfg = _model(2)
    ids = _steps(SEQS, 2)
    state = ML.forward_full(p, cfg, ids[0], SEQS)
    off, n, bs, be = SEQS[0]
    rng = np.random.default_rng(3)
    xb = round_bf16(rng.standard_normal((be - bs, D)))
    lp = p["layers"][1]
    qb, kb, vb = ML.layer_qkv(xb, lp, cfg, np.arange(bs, be))
    k = state["K"][1][off:off + n].copy()
    v = state["V"][1][off:off + n].copy()
    k[bs:be], v[bs:be] = kb, vb
    got = ML.layer_attention(qb, k, v, cfg)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))       # [H, N, d]
    ref = F.scaled_dot_product_attention(t(qb), t(k), t(v)).numpy().transpose(1, 0, 2).reshape(be - bs, -1)
    np.testing.assert_allclose(got, round_bf16(ref), rtol=2 ** -7, atol=1e-12)
