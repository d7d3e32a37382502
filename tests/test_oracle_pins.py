"""Pins of the fp64 oracle against things other than itself.

Each test checks one part of the oracle against a library routine, a closed
form, a hand-worked value or a scalar brute force, so that a dropped term, a
wrong sign or index, or a transposed operand in the oracle fails at least one
of them.  No GPU is used.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import Layer0Config
from exact_attention_state_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rng(*s):
    return np.random.default_rng([7, *s])


# ---------------------------------------------------------------- RMSNorm ---

def test_rms_norm_matches_torch_rms_norm():
    r = _rng(1)
    H = r.standard_normal((9, 37)) * 3
    g = 1 + 0.3 * r.standard_normal(37)
    for eps in (1e-5, 0.5):
        ref = F.rms_norm(torch.from_numpy(H), (37,), torch.from_numpy(g), eps=eps).numpy()
        np.testing.assert_allclose(oracle.rms_norm(H, g, eps), ref, rtol=1e-13, atol=1e-13)


def test_rms_norm_unit_gain_closed_form():
    # gamma = 1: the output's mean square is ms / (ms + eps).
    r = _rng(2)
    H = r.standard_normal((5, 64)) * 0.01
    eps = 1e-5
    ms = np.mean(H * H, axis=1)
    out = oracle.rms_norm(H, np.ones(64), eps)
    np.testing.assert_allclose(np.mean(out * out, axis=1), ms / (ms + eps), rtol=1e-12)


# ------------------------------------------------------------------- RoPE ---

def test_rope_hand_worked_example():
    # d_h = 4, theta = 100 -> inverse frequencies 1 and 100^(-1/2) = 0.1.
    # Position 2: features (0, 2) rotate by 2 rad, features (1, 3) by 0.2 rad.
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    got = oracle.rope(x, np.array([2]), 100.0)[0, 0]
    want = [1 * math.cos(2) - 3 * math.sin(2), 2 * math.cos(0.2) - 4 * math.sin(0.2),
            1 * math.sin(2) + 3 * math.cos(2), 2 * math.sin(0.2) + 4 * math.cos(0.2)]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_is_complex_rotation():
    # Pair (x_i, x_{i+d/2}) as z = x_i + j x_{i+d/2}; RoPE multiplies z by e^{j p w_i}.
    r = _rng(3)
    d, theta = 16, 5e5
    x = r.standard_normal((11, 3, d))
    pos = r.integers(0, 5000, size=11)
    w = np.array([theta ** (-(2.0 * i) / d) for i in range(d // 2)])
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * w[None, None, :])
    got = oracle.rope(x, pos, theta)
    np.testing.assert_allclose(got[..., : d // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(got[..., d // 2:], z.imag, atol=1e-12)


def test_rope_position_zero_is_identity_and_norms_preserved():
    r = _rng(4)
    x = r.standard_normal((6, 2, 8))
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(6, int), 1e4), x)
    y = oracle.rope(x, np.arange(6) * 977, 1e4)
    np.testing.assert_allclose(np.hypot(y[..., :4], y[..., 4:]), np.hypot(x[..., :4], x[..., 4:]), rtol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    r = _rng(5)
    q = r.standard_normal((1, 1, 32)); k = r.standard_normal((1, 1, 32))
    s = [float(oracle.rope(q, np.array([10 + c]), 1e4)[0, 0] @ oracle.rope(k, np.array([3 + c]), 1e4)[0, 0])
         for c in (0, 17, 1000)]
    np.testing.assert_allclose(s, s[0], rtol=1e-11)


def test_rope_block_offset_equals_slice_of_full_sequence():
    # decode_block(..., block_start) "for correct RoPE offset": a block alone at
    # positions bs.. equals the same rows of RoPE applied to the full sequence.
    r = _rng(6)
    x = r.standard_normal((40, 2, 8))
    full = oracle.rope(x, np.arange(40), 1e4)
    np.testing.assert_array_equal(oracle.rope(x[24:32], np.arange(24, 32), 1e4), full[24:32])


# -------------------------------------------------------------- attention ---

def test_attention_matches_torch_sdpa_and_logsumexp():
    r = _rng(7)
    q, k, v = r.standard_normal((13, 16)), r.standard_normal((29, 16)), r.standard_normal((29, 16))
    O, lse = oracle.attention(q, k, v, 1 / 4.0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(q @ k.T / 4.0, axis=1), rtol=1e-13)


def test_merge_of_partial_states_equals_softmax_over_union():
    r = _rng(8)
    q, k, v = r.standard_normal((7, 8)), 3 * r.standard_normal((20, 8)), r.standard_normal((20, 8))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], scale=0.7)[0].numpy()
    ref_lse = scipy.special.logsumexp(0.7 * q @ k.T, axis=1)
    for split in (0, 1, 9, 19, 20):          # includes empty sides
        perm = r.permutation(20)
        a, b = perm[:split], perm[split:]
        st = oracle.merge_states(oracle.state_over_keys(q, k[a], v[a], 0.7),
                                 oracle.state_over_keys(q, k[b], v[b], 0.7))
        O, lse = oracle.finalize(st)
        np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


def test_online_update_stream_equals_softmax():
    # Eqs. (2)-(6) streamed tile by tile from the empty state give softmax attention.
    r = _rng(9)
    q, k, v = r.standard_normal((5, 8)), 4 * r.standard_normal((23, 8)), r.standard_normal((23, 8))
    st = (np.full(5, -np.inf), np.zeros(5), np.zeros((5, 8)))
    for j in range(0, 23, 6):
        st = oracle.online_update(st, q, k[j:j + 6], v[j:j + 6], 0.35)
    O, lse = oracle.finalize(st)
    p = scipy.special.softmax(0.35 * q @ k.T, axis=1)
    np.testing.assert_allclose(O, p @ v, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(0.35 * q @ k.T, axis=1), rtol=1e-13)


# ------------------------------------------------------- layer 0 / caches ---

def _tiny_params(r, V, D, F_, eps_scale=1.0):
    return {"embed": r.standard_normal((V, D)) * eps_scale, "gamma": 1 + 0.2 * r.standard_normal(D),
            "w_qkv": 0.3 * r.standard_normal((F_, D))}


def _brute_layer0(params, cfg, ids_b):
    """Scalar loops over one sequence: embed, RMSNorm, QKV, RoPE, softmax attention."""
    N, D, H, Hk, d = len(ids_b), cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    E, g, W = params["embed"], params["gamma"], params["w_qkv"]
    q = [[[0.0] * d for _ in range(H)] for _ in range(N)]
    k = [[[0.0] * d for _ in range(Hk)] for _ in range(N)]
    v = [[[0.0] * d for _ in range(Hk)] for _ in range(N)]
    for t in range(N):
        row = [float(E[ids_b[t]][c]) for c in range(D)]
        rms = math.sqrt(sum(x * x for x in row) / D + cfg.rms_eps)
        hh = [float(g[c]) * row[c] / rms for c in range(D)]
        feats = [sum(float(W[f][c]) * hh[c] for c in range(D)) for f in range(W.shape[0])]
        for hd in range(H):
            q[t][hd] = feats[hd * d:(hd + 1) * d]
        for hd in range(Hk):
            k[t][hd] = feats[(H + hd) * d:(H + hd + 1) * d]
            v[t][hd] = feats[(H + Hk + hd) * d:(H + Hk + hd + 1) * d]
        for vec_list in (q[t], k[t]):
            for vec in vec_list:
                old = list(vec)
                for i in range(d // 2):
                    ang = t * cfg.rope_theta ** (-2.0 * i / d)
                    vec[i] = old[i] * math.cos(ang) - old[i + d // 2] * math.sin(ang)
                    vec[i + d // 2] = old[i] * math.sin(ang) + old[i + d // 2] * math.cos(ang)
    out = np.zeros((N, H, d)); lse = np.zeros((N, H))
    grp = H // Hk
    for hd in range(H):
        kh = hd // grp
        for t in range(N):
            s = [cfg.scale * sum(q[t][hd][c] * k[j][kh][c] for c in range(d)) for j in range(N)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = sum(w)
            for c in range(d):
                out[t, hd, c] = sum(w[j] * v[j][kh][c] for j in range(N)) / tot
            lse[t, hd] = mx + math.log(tot)
    return out, lse, np.array(q), np.array(k), np.array(v)


@pytest.mark.parametrize("H,Hk", [(2, 2), (2, 1)])
def test_full_recompute_matches_scalar_brute_force(H, Hk):
    r = _rng(10, H, Hk)
    cfg = Layer0Config(d_model=16, n_heads=H, n_kv_heads=Hk, head_dim=8, rope_theta=10.0, rms_eps=1e-5)
    params = _tiny_params(r, 23, 16, cfg.n_features)
    seqs = [(0, 8, 2, 6), (8, 5, 4, 5)]
    ids = r.integers(0, 23, size=13)
    res = oracle.full_recompute(params, cfg, ids, seqs)
    for (off, n, _, _) in seqs:
        out, lse, q, k, v = _brute_layer0(params, cfg, ids[off:off + n])
        np.testing.assert_allclose(res["out"][off:off + n], out, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["lse"][off:off + n], lse, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["q"][off:off + n], q, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["k"][off:off + n], k, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(res["v"][off:off + n], v, rtol=1e-11, atol=1e-12)


def test_attention_part_matches_sdpa_per_sample_and_head():
    # Keys never cross samples; grouped KV heads are shared by consecutive query heads.
    r = _rng(11)
    cfg = Layer0Config(d_model=32, n_heads=4, n_kv_heads=2, head_dim=8, rope_theta=1e4)
    params = _tiny_params(r, 50, 32, cfg.n_features)
    seqs = [(0, 17, 3, 9), (17, 30, 20, 28)]
    ids = r.integers(0, 50, size=47)
    res = oracle.full_recompute(params, cfg, ids, seqs)
    for (off, n, _, _) in seqs:
        sl = slice(off, off + n)
        q = torch.from_numpy(res["q"][sl]).permute(1, 0, 2)
        k = torch.from_numpy(res["k"][sl]).permute(1, 0, 2).repeat_interleave(2, dim=0)
        v = torch.from_numpy(res["v"][sl]).permute(1, 0, 2).repeat_interleave(2, dim=0)
        ref = F.scaled_dot_product_attention(q, k, v).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(res["out"][sl], ref, rtol=1e-12, atol=1e-13)


def test_facache_state_matches_masked_sdpa():
    # FACache = online state of invariant rows over invariant keys only.
    r = _rng(12)
    cfg = Layer0Config(d_model=32, n_heads=2, n_kv_heads=2, head_dim=8, rope_theta=1e4)
    params = _tiny_params(r, 40, 32, cfg.n_features)
    seqs = [(0, 21, 8, 12)]
    ids = r.integers(0, 40, size=21)
    res = oracle.refresh(params, cfg, ids, seqs)
    U = np.r_[0:8, 12:21]
    mask = torch.zeros(21, 21, dtype=torch.bool)
    mask[:, torch.from_numpy(U)] = True
    q = torch.from_numpy(res["q"]).permute(1, 0, 2)
    k = torch.from_numpy(res["k"]).permute(1, 0, 2)
    v = torch.from_numpy(res["v"]).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask).permute(1, 0, 2).numpy()
    s = np.einsum("hid,hjd->hij", q.numpy(), k.numpy()) / math.sqrt(8)
    ref_lse = scipy.special.logsumexp(s[:, :, U], axis=2).T
    np.testing.assert_allclose(res["o_c"][U] / res["l_c"][U][..., None], ref[U], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res["m_c"][U] + np.log(res["l_c"][U]), ref_lse[U], rtol=1e-13)
    assert np.isnan(res["m_c"][8:12]).all()


def test_zero_key_weights_closed_form():
    # W_K = 0 -> every score is 0: O = mean of v over the sequence, LSE = log N,
    # FACache = (0, |U|, sum of v over U).
    r = _rng(13)
    cfg = Layer0Config(d_model=16, n_heads=2, n_kv_heads=2, head_dim=8, rope_theta=1e4)
    params = _tiny_params(r, 30, 16, cfg.n_features)
    params["w_qkv"][16:32] = 0.0
    seqs = [(0, 12, 4, 8)]
    ids = r.integers(0, 30, size=12)
    res = oracle.refresh(params, cfg, ids, seqs)
    np.testing.assert_allclose(res["out"], np.broadcast_to(res["v"].mean(axis=0), res["out"].shape), atol=1e-13)
    np.testing.assert_allclose(res["lse"], math.log(12), rtol=1e-14)
    U = np.r_[0:4, 8:12]
    np.testing.assert_array_equal(res["m_c"][U], 0.0)
    np.testing.assert_allclose(res["l_c"][U], 8.0, rtol=1e-14)
    np.testing.assert_allclose(res["o_c"][U], np.broadcast_to(res["v"][U].sum(axis=0), (8, 2, 8)), atol=1e-12)


def _run_steps(wl, params, cfg, nsteps):
    seqs = wl.table()
    ids = synth.initial_ids(wl)
    cache = oracle.refresh(params, cfg, ids, seqs)
    for s in range(1, nsteps + 1):
        ids, blk = synth.step_ids(wl, ids, s)
        got = oracle.cached_step(params, cfg, cache, blk, seqs, kv_tile=5)
        want = oracle.full_recompute(params, cfg, ids, seqs)
        yield got, want
        cache.update({k: got[k] for k in ("h", "q", "k", "v")})


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged"])
def test_cached_step_equals_full_recompute(name):
    # The method's claim: the cached step's output equals the full recompute.
    if name == "tiny":
        wl = synth.WORKLOADS["tiny"]
    else:
        wl = synth.custom("gqa_ragged", dtype="f32", d_model=64, n_heads=4, n_kv_heads=2, head_dim=16,
                          vocab=97, prompt_lens=(5, 23, 0), gen_len=21, block_size=7, steps=3, seed=11)
    params = synth.params(wl)
    cfg = Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)
    for got, want in _run_steps(wl, params, cfg, wl.steps):
        for key in ("h", "q", "k", "v", "out", "lse"):
            np.testing.assert_allclose(got[key], want[key], rtol=1e-10, atol=1e-12, err_msg=key)


def test_cached_step_without_refresh_is_wrong():
    # Negative control: reusing the FACache of another block's layout breaks exactness.
    wl = synth.WORKLOADS["tiny"]
    params = synth.params(wl)
    cfg = Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)
    seqs = wl.table()
    ids = synth.initial_ids(wl)
    stale = oracle.refresh(params, cfg, ids, [(0, 128, 64, 80)])      # cache for block 0
    blk = synth.block_ids_of(wl, ids)
    got = oracle.cached_step(params, cfg, stale, blk, seqs)
    want = oracle.full_recompute(params, cfg, ids, seqs)
    assert np.nanmax(np.abs(got["out"] - want["out"])) > 1e-6


def test_u_empty_block_covers_whole_sequence():
    # N = B: no invariant rows; the step is plain attention over the block.
    r = _rng(14)
    cfg = Layer0Config(d_model=16, n_heads=2, n_kv_heads=2, head_dim=8, rope_theta=1e4)
    params = _tiny_params(r, 30, 16, cfg.n_features)
    seqs = [(0, 6, 0, 6)]
    ids = r.integers(0, 30, size=6)
    cache = oracle.refresh(params, cfg, ids, seqs)
    assert np.isnan(cache["m_c"]).all()
    got = oracle.cached_step(params, cfg, cache, ids, seqs)
    np.testing.assert_allclose(got["out"], cache["out"], rtol=1e-13)


def test_layer0_rows_matches_full_sample():
    wl = synth.custom("rows", dtype="f32", d_model=64, n_heads=4, n_kv_heads=2, head_dim=16,
                      vocab=80, prompt_lens=(30,), gen_len=16, block_size=8, seed=12)
    params = synth.params(wl)
    cfg = Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)
    ids = synth.initial_ids(wl)
    full = oracle.layer0_sample(params, cfg, ids)
    rows, heads = [0, 7, 45, 31], [3, 0]
    part = oracle.layer0_rows(params, cfg, ids, rows, heads)
    np.testing.assert_allclose(part["out"], full["out"][rows][:, heads], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(part["lse"], full["lse"][rows][:, heads], rtol=1e-13)


def test_oracle_regression_fixture():
    # Drift guard only (written by tests/golden/make_golden.py from the oracle).
    import json
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_samples.json")) as f:
        want = json.load(f)
    got = make_golden.build()
    for key in want:
        if key == "workload":
            assert got[key] == want[key]
            continue
        np.testing.assert_allclose(np.asarray(got[key], dtype=float), np.asarray(want[key], dtype=float),
                                   rtol=1e-12, atol=1e-14, err_msg=key)
