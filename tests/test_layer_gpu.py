"""GPU parity of the rest of layer 0 (lacache_layer_finish) and of the sampler
cut (lacache_sampler_cut) with the layer oracle (oracle/layer_ref.py).

Every stage is checked from the GPU's own inputs to that stage (the
workspace holds x, y, z and the logits), against the oracle's fp64 value of
the stage and the rounding its reading prescribes:
* a bf16 output must be the rounding of some value within the stage's error
  bound of the exact one: fp32 accumulation over K products of bf16 values,
  at most K 2^-24 sum |a_k b_k| (RMSNorm: 2^-16 relative for the fp32 sum of
  squares and reciprocal root; SwiGLU: the four roundings of gate and up
  that bound allows, and 2^-20 relative for the fp32 silu), and most outputs
  must equal the oracle's rounding of the exact value;
* the logits (fp32, unrounded) within that bound; the token must be an
  argmax of the exact logits within twice the bound; the confidence and the
  probabilities against the softmax of the GPU's own logits (1e-5 relative).
The cut is checked to equal the uncut sampler on the block rows, bit for bit.
"""

import os
import sys

import numpy as np
import pytest
import torch

from oracle import layer_ref as L
from oracle.fp8_ref import round_bf16
from exact_attention_state_amd import lacache, synth

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _ctx(D, H, max_seq=4096):
    return lacache.Context(D, H, H, 128, 1000, max_seq, 1e4, 1e-5, 0.0, "bf16")


def _dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dtype).cuda()


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _ws_bf16(ws, offset, n, d):
    return _np(ws[offset:offset + n * d * 2].view(torch.bfloat16).reshape(n, d))


def _a256(x):
    return (x + 255) // 256 * 256


def _check_rounded(got, exact, err, what, min_equal=0.99):
    """got: a bf16 rounding of a value in [exact - err, exact + err]; most equal to round(exact)."""
    lo, hi = round_bf16(exact - err), round_bf16(exact + err)
    bad = ~((got >= lo) & (got <= hi))
    assert not bad.any(), f"{what}: {bad.sum()} outside the bound, e.g. got {got[bad][:4]} exact {exact[bad][:4]}"
    eq = float(np.mean(got == round_bf16(exact)))
    _say(f"  {what}: all within the bound, {eq:.5f} equal to the oracle's rounding")
    assert eq >= min_equal, f"{what}: only {eq} equal to the oracle's rounding"


def _check_chain(got, base, inner_exact, inner_err, what, min_equal=0.99):
    """got = bf16(base + bf16(inner)) with inner within inner_err of inner_exact."""
    lo = round_bf16(base + round_bf16(inner_exact - inner_err))
    hi = round_bf16(base + round_bf16(inner_exact + inner_err))
    bad = ~((got >= lo) & (got <= hi))
    assert not bad.any(), f"{what}: {bad.sum()} outside the bound"
    eq = float(np.mean(got == round_bf16(base + round_bf16(inner_exact))))
    _say(f"  {what}: all within the bound, {eq:.5f} equal to the oracle's rounding")
    assert eq >= min_equal


def _lin_err(x, w):
    return x.shape[1] * U24 * (np.abs(x) @ np.abs(w).T) + 1e-30


def _check_layer_rows(rows, h, o, w, r, x, y, out, D, F):
    """Stage checks of lacache_layer_finish on the given rows (GPU values r, x, y, out)."""
    w_o, g, wg, wu, wd = w
    h, o, r, x, y, out = h[rows], o[rows], r[rows], x[rows], y[rows], out[rows]
    # r = bf16(h + bf16(O W_o^T))
    _check_chain(r, h, L.linear(o, w_o), _lin_err(o, w_o), "r")
    # x = bf16(RMSNorm(r)) from the GPU's r
    xe = L.rms_norm_rows(r, g, 1e-5)
    _check_rounded(x, xe, np.abs(xe) * 2.0 ** -16, "x")
    # y = bf16(silu(bf16(gate)) bf16(up)) from the GPU's x
    ge, ue = L.linear(x, wg), L.linear(x, wu)
    eg, eu = _lin_err(x, wg), _lin_err(x, wu)
    cands = []
    for gg in (round_bf16(ge - eg), round_bf16(ge + eg)):
        for uu in (round_bf16(ue - eu), round_bf16(ue + eu)):
            cands.append(gg / (1.0 + np.exp(-gg)) * uu)
    cands = np.stack(cands)
    ylo, yhi = cands.min(0), cands.max(0)
    ylo, yhi = ylo - np.abs(ylo) * 2.0 ** -20, yhi + np.abs(yhi) * 2.0 ** -20
    bad = ~((y >= round_bf16(ylo)) & (y <= round_bf16(yhi)))
    assert not bad.any(), f"y: {bad.sum()} outside the bound"
    yref = round_bf16(L.silu(round_bf16(ge)) * round_bf16(ue))
    eqy = float(np.mean(y == yref))
    _say(f"  y: all within the bound, {eqy:.5f} equal to the oracle's rounding")
    assert eqy >= 0.99
    # out = bf16(r + bf16(y W_d^T)) from the GPU's y and r
    _check_chain(out, r, L.linear(y, wd), _lin_err(y, wd), "out")


def _run_layer(D, H, F, T, seed, tile=None, monkeypatch=None):
    if tile and monkeypatch:
        monkeypatch.setenv("LACACHE_LAYER_TILE", tile)
    ctx = _ctx(D, H)
    HD = H * 128
    p = synth.layer_params(D, HD, F, seed)
    h, o = synth.ffn_inputs(T, D, seed)[0], synth.ffn_inputs(T, HD, seed + 1)[1]
    wts = [p["w_o"], p["gamma"], p["w_gate"], p["w_up"], p["w_down"]]
    dw = [_dev(t) for t in wts]
    hd, od = _dev(h), _dev(o)
    out = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    r = torch.empty_like(out)
    ws = ctx.layer_workspace(F, T, True)
    ws.fill_(0)
    ctx.layer_finish(F, dw, hd, od, out, r_out=r, workspace=ws)
    torch.cuda.synchronize()
    assert ctx.read_device_status() == 0
    x = _ws_bf16(ws, 0, T, D)
    y = _ws_bf16(ws, _a256(T * D * 2), T, F)
    return ctx, (h, o), [w.astype(np.float64) for w in wts], _np(r), x, y, _np(out)


# Up to 64 rows with few output tiles the GEMMs split their contraction
# (partials reduced in a second kernel): 1, 17, 32, 61 and 64 rows, and
# LLaDA-8B's layer shape at a block of 32 rows (16 splits of W_o and down).
# More rows with few 128 x 128 tiles and a long contraction split the down
# projection too: d_ff 6144 (two splits) and 12288 (four), at 300 and 200
# rows, and at 40 rows with the 128 x 128 tiles forced.
@pytest.mark.parametrize("D,H,F,T,tile", [(512, 4, 384, 77, None), (1024, 8, 512, 300, None),
                                           (512, 4, 6144, 300, None), (512, 4, 12288, 200, None),
                                           (1024, 8, 12288, 40, "128"),
                                           (512, 4, 384, 513, "256"), (512, 4, 256, 200, "128"),
                                           (512, 4, 256, 130, "64"), (512, 4, 256, 200, "128w4"),
                                           (512, 4, 384, 1, None),
                                           (1024, 8, 512, 17, None), (1024, 8, 768, 61, None),
                                           (1024, 8, 512, 64, None), (4096, 32, 12288, 32, None)])
def test_layer_finish_every_row(D, H, F, T, tile, monkeypatch):
    _say(f"[layer] D {D} heads {H} d_ff {F} rows {T} tile {tile}")
    ctx, (h, o), w, r, x, y, out = _run_layer(D, H, F, T, 3, tile, monkeypatch)
    _check_layer_rows(np.arange(T), h.astype(np.float64), o.astype(np.float64), w, r, x, y, out, D, F)
    # end to end against the oracle's own chain
    ref = L.layer0_finish(h, o, *w, 1e-5)
    rel = np.linalg.norm(out - ref["out"], axis=1) / np.linalg.norm(ref["out"], axis=1)
    _say(f"  end to end: max row error {rel.max():.2e}")
    assert rel.max() < 1e-2


def _sampler_check(ctx, hidden, table, gf, w_lm, token, conf, probs, ws, D, V):
    rows = L.block_rows(table)
    M = len(rows)
    z = _ws_bf16(ws, 0, M, D)
    ze = L.rms_norm_rows(hidden[rows], gf, 1e-5)
    _check_rounded(z, ze, np.abs(ze) * 2.0 ** -16, "z")
    lg = ws[_a256(M * D * 2):_a256(M * D * 2) + M * V * 4].view(torch.float32).reshape(M, V).double().cpu().numpy()
    le = np.empty((M, V))
    err = np.empty((M, V))
    for v0 in range(0, V, 4096):                        # the lm-head in slices of the vocabulary
        wv = w_lm[v0:v0 + 4096].astype(np.float64)
        le[:, v0:v0 + 4096] = z @ wv.T
        err[:, v0:v0 + 4096] = (D + 1) * U24 * (np.abs(z) @ np.abs(wv).T) + 1e-30
    bad = np.abs(lg - le) > err
    assert not bad.any(), f"logits: {bad.sum()} outside the bound"
    tok = token.cpu().numpy()
    emax = le.max(1)
    assert np.all(le[np.arange(M), tok] >= emax - 2 * err.max(1)), "token is not an argmax of the exact logits"
    eq_tok = float(np.mean(tok == np.argmax(le, 1)))
    p_gpu = np.exp(lg - lg.max(1, keepdims=True))
    p_gpu /= p_gpu.sum(1, keepdims=True)
    np.testing.assert_allclose(conf.cpu().numpy(), p_gpu[np.arange(M), tok], rtol=1e-5)
    assert np.all(tok == np.argmax(lg, 1)), "token is not the first argmax of the GPU's logits"
    if probs is not None:
        np.testing.assert_allclose(probs.cpu().numpy().reshape(M, V), p_gpu, rtol=1e-5, atol=1e-12)
    _say(f"  sampler: {M} rows, logits within the bound, tokens equal to the oracle's argmax {eq_tok:.4f}")


@pytest.mark.parametrize("D,V,tile", [(512, 1000, None), (1024, 4104, "256"), (512, 2048, "128")])
def test_sampler_cut_matches_oracle_and_uncut(D, V, tile, monkeypatch):
    _say(f"[sampler] D {D} vocab {V} tile {tile}")
    if tile:
        monkeypatch.setenv("LACACHE_LAYER_TILE", tile)
    ctx = _ctx(D, D // 128)
    table = [(0, 120, 16, 32), (120, 300, 200, 232), (420, 50, 43, 50)]
    n_rows = 470
    rng = np.random.default_rng([31, D, V])
    hidden = round_bf16(rng.standard_normal((n_rows, D))).astype(np.float32)
    p = synth.lm_head_params(D, V, 1)
    hd, gd, wd = _dev(hidden), _dev(p["gamma_f"]), _dev(p["w_lm"])
    M = sum(be - bs for _, _, bs, be in table)
    token = torch.empty(M, dtype=torch.int32, device="cuda")
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    probs = torch.empty(M, V, dtype=torch.float32, device="cuda")
    ws = ctx.sampler_workspace(V, table)
    ctx.sampler_cut(hd, table, gd, wd, token, conf, probs, workspace=ws)
    torch.cuda.synchronize()
    _sampler_check(ctx, hidden.astype(np.float64), table, p["gamma_f"].astype(np.float64), p["w_lm"], token, conf,
                   probs, ws, D, V)
    # the uncut sampler (every row of every sequence) agrees on the block rows, bit for bit
    full = [(off, n, 0, n) for off, n, _, _ in table]
    Mf = sum(n for _, n, _, _ in full)
    tf = torch.empty(Mf, dtype=torch.int32, device="cuda")
    cf = torch.empty(Mf, dtype=torch.float32, device="cuda")
    ctx.sampler_cut(hd, full, gd, wd, tf, cf)
    torch.cuda.synchronize()
    sel = np.concatenate([np.arange(o_ + bs, o_ + be) for (o_, _, bs, be) in table])
    # rows of the full table are in table order: offset o_ .. o_ + n, so row index = global row here
    assert torch.equal(tf[torch.from_numpy(sel).cuda()], token)
    assert torch.equal(cf[torch.from_numpy(sel).cuda()], conf)


def test_layer_and_sampler_llada8b_from_a_block_step():
    """llada8b: the layer finish on the attention output of a real block step
    (768 rows, d_model 4096, 32 heads x 128, d_ff 12288), then the sampler cut
    (vocabulary 126464) on the block's 32 rows; sampled rows checked stage by
    stage, the sampler on every block row."""
    from exact_attention_state_amd.workload import DeviceWorkload
    wl = synth.WORKLOADS["llada8b"]
    _say("[layer] llada8b: block step, layer finish, sampler cut")
    dw = DeviceWorkload(wl, device="cuda")
    dw.prefill()
    dw.block_step(dw.next_block_ids())
    torch.cuda.synchronize()
    T, D, F, V = wl.total_tokens, wl.d_model, synth.LLADA_D_FF, synth.LLADA_VOCAB
    HD = wl.n_heads * wl.head_dim
    h = dw.ct.h.reshape(T, D)
    o = dw.ct.out.reshape(T, HD)
    p = synth.layer_params(D, HD, F, 0)
    wts = [p["w_o"], p["gamma"], p["w_gate"], p["w_up"], p["w_down"]]
    dws = [_dev(t) for t in wts]
    out = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    r = torch.empty_like(out)
    ws = dw.ctx.layer_workspace(F, T, True)
    dw.ctx.layer_finish(F, dws, h, o, out, r_out=r, workspace=ws)
    torch.cuda.synchronize()
    x = _ws_bf16(ws, 0, T, D)
    y = _ws_bf16(ws, _a256(T * D * 2), T, F)
    bs = dw.table[0][2]
    rows = np.array([0, 1, 300, bs, bs + 7, bs + 31, T - 2, T - 1])
    _check_layer_rows(rows, _np(h), _np(o), [w_.astype(np.float64) for w_ in wts], _np(r), x, y, _np(out), D, F)
    del dws, ws
    lm = synth.lm_head_params(D, V, 0)
    gd, wd = _dev(lm["gamma_f"]), _dev(lm["w_lm"])
    M = sum(be - bs_ for _, _, bs_, be in dw.table)
    token = torch.empty(M, dtype=torch.int32, device="cuda")
    conf = torch.empty(M, dtype=torch.float32, device="cuda")
    sws = dw.ctx.sampler_workspace(V, dw.table)
    dw.ctx.sampler_cut(out, dw.table, gd, wd, token, conf, workspace=sws)
    torch.cuda.synchronize()
    _sampler_check(dw.ctx, _np(out), dw.table, lm["gamma_f"].astype(np.float64), lm["w_lm"], token, conf, None, sws,
                   D, V)
    assert dw.ctx.read_device_status() == 0


def test_layer_and_sampler_reject_bad_arguments():
    ctx = _ctx(512, 4)
    w = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in ((512, 512), (512,), (384, 512), (384, 512),
                                                                      (512, 384))]
    h = torch.zeros(16, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lacache.LaCacheError):                      # d_ff not a multiple of 128
        ctx.layer_finish(300, w, h, h, h.clone())
    with pytest.raises(lacache.LaCacheError):                      # workspace too small
        ctx.layer_finish(384, w, h, h, h.clone(), workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    wl = torch.zeros(1000, 512, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(512, dtype=torch.bfloat16, device="cuda")
    tok = torch.empty(8, dtype=torch.int32, device="cuda")
    cf = torch.empty(8, dtype=torch.float32, device="cuda")
    with pytest.raises(lacache.LaCacheError):                      # rows past the hidden buffer
        ctx.sampler_cut(h, [(10, 8, 0, 8)], g, wl, tok, cf)
    with pytest.raises(lacache.LaCacheError):                      # vocabulary not a multiple of 8
        ctx.sampler_cut(h, [(0, 8, 0, 8)], g, wl[:999], tok, cf)
