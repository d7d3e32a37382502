"""Planted mistakes in the oracle must fail its pins.

Each mutation below replaces one oracle function with a plausibly wrong
version (a dropped term, a wrong sign, index, base, rounding or operand
order); with it in place, at least one pin of tests/test_oracle_pins.py,
tests/test_fp8_oracle_pins.py, tests/test_layer_oracle_pins.py,
tests/test_multilayer_oracle_pins.py or tests/test_flashdllm_oracle_pins.py
other than the regression fixture (which the oracle itself wrote) must fail.  The mistakes
are planted in the oracle on the CPU only; no GPU is used.
"""

import numpy as np
import pytest

import oracle
import oracle.fp8_ref as q8
import oracle.lacache_ref as ref
import oracle.layer_ref as lay
import oracle.multilayer_ref as mlr
import oracle.flashdllm_ref as fdr
import test_flashdllm_oracle_pins as fd_pins
import test_fp8_oracle_pins as fp8_pins
import test_layer_oracle_pins as layer_pins
import test_multilayer_oracle_pins as ml_pins
import test_oracle_pins as pins


def _pin_calls():
    """Every pin as a zero-argument call (parametrized pins expanded)."""
    calls = []
    for mod, name in sorted([(p, n) for p in (pins, fp8_pins, layer_pins, ml_pins, fd_pins) for n in dir(p)], key=lambda x: x[1]):
        fn = getattr(mod, name)
        if not name.startswith("test_") or not callable(fn) or name == "test_oracle_regression_fixture":
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        combos = [{}]
        for m in params:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            new = []
            for c in combos:
                for vals in m.args[1]:
                    vals = vals if len(argnames) > 1 else (vals,)
                    new.append({**c, **dict(zip(argnames, vals))})
            combos = new
        calls.extend((f"{name}{c}", fn, c) for c in combos)
    return calls


# ---------------------------------------------------------------- mutants ---

def _rms_no_gamma(H, gamma, eps):
    H = np.asarray(H, np.float64)
    return H / np.sqrt(np.mean(H * H, axis=-1, keepdims=True) + eps)


def _rms_eps_outside(H, gamma, eps):
    H = np.asarray(H, np.float64)
    return np.asarray(gamma, np.float64) * H / (np.sqrt(np.mean(H * H, axis=-1, keepdims=True)) + eps)


def _qkv_k_v_swapped(Hhat, W, cfg):
    q, k, v = ref.__dict__["_orig_qkv_project"](Hhat, W, cfg)
    return q, v, k


def _qkv_heads_feature_major(Hhat, W, cfg):
    y = np.asarray(Hhat, np.float64) @ np.asarray(W, np.float64).T
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    q = y[:, : H * d].reshape(-1, d, H).transpose(0, 2, 1)
    k = y[:, H * d: (H + Hk) * d].reshape(-1, Hk, d)
    v = y[:, (H + Hk) * d:].reshape(-1, Hk, d)
    return q, k, v


def _rope_angles_half_freq(pos, head_dim, theta):
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.asarray(pos, np.float64)[:, None] * np.power(float(theta), -1.0 * i / head_dim)[None, :]


def _rope_wrong_sign(x, pos, theta):
    x = np.asarray(x, np.float64)
    half = x.shape[-1] // 2
    ang = ref.rope_angles(pos, x.shape[-1], theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def _finalize_log2(state):
    m, l, O = state
    return O / l[:, None], m + np.log2(l)


def _online_alpha_inverted(state, q, k_tile, v_tile, scale):
    m, l, O = state
    S = scale * (np.asarray(q, np.float64) @ np.asarray(k_tile, np.float64).T)
    m_new = np.maximum(m, S.max(axis=1))
    with np.errstate(invalid="ignore", over="ignore"):
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m_new - m))
    P = np.exp(S - m_new[:, None])
    return m_new, alpha * l + P.sum(axis=1), alpha[:, None] * O + P @ np.asarray(v_tile, np.float64)


def _merge_unscaled_second(s1, s2):
    m1, l1, O1 = s1
    m2, l2, O2 = s2
    m = np.maximum(m1, m2)
    with np.errstate(invalid="ignore"):
        a1 = np.where(np.isneginf(m1), 0.0, np.exp(m1 - m))
    return m, a1 * l1 + l2, a1[:, None] * O1 + O2


def _facache_all_keys(q, k, v, U, cfg):
    H, d = cfg.n_heads, cfg.head_dim
    n = len(q)
    m = np.empty((len(U), H)); l = np.empty((len(U), H)); O = np.empty((len(U), H, d))
    for hd in range(H):
        kh = ref._kv_head(hd, cfg)
        m[:, hd], l[:, hd], O[:, hd] = ref.state_over_keys(q[U, hd], k[np.arange(n), kh], v[np.arange(n), kh],
                                                           cfg.scale)
    return (m, l, O), (O / l[..., None], m + np.log(l))


def _kv_head_modulo(h, cfg):
    return h % cfg.n_kv_heads


def _attention_unscaled(q, k, v, scale):
    return ref.__dict__["_orig_attention"](q, k, v, 1.0)


def _cached_step_block_at_zero(params, cfg, cache, block_ids, seqs, kv_tile=16):
    # RoPE of the block computed at positions 0..B-1 instead of block_start..
    orig_rope = ref.rope

    def rope_from_zero(x, pos, theta):
        pos = np.asarray(pos)
        if len(pos) and len(pos) == len(x) and pos[0] > 0 and np.all(np.diff(pos) == 1) and len(pos) < 64:
            pos = pos - pos[0]
        return orig_rope(x, pos, theta)

    ref.rope = rope_from_zero
    try:
        return ref.__dict__["_orig_cached_step"](params, cfg, cache, block_ids, seqs, kv_tile)
    finally:
        ref.rope = orig_rope


def _round_e4m3_toward_zero(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    idx = np.searchsorted(q8._POS, a, side="right") - 1
    return np.copysign(q8._POS[idx], v)


def _round_e4m3_ties_away(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    hi = np.minimum(np.searchsorted(q8._POS, a, side="left"), len(q8._POS) - 1)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (q8._POS[hi] - a) <= (a - q8._POS[lo])
    return np.copysign(np.where(pick_hi, q8._POS[hi], q8._POS[lo]), v)


def _quantize_group_scale_times(x32, amax32):
    # scale = amax * Q_max instead of amax / Q_max
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = (amax32 * np.float32(q8.E4M3_MAX)).astype(np.float32)
        v = np.where(scale == 0, 0, x32 / scale)
    return q8.round_e4m3(np.clip(v, -448, 448)), scale


def _quantize_weight_row_stripes(w, group=128):
    # one scale per 128 rows over the whole contraction, not per 128 x 128 block
    w32 = np.asarray(w, np.float64).astype(np.float32)
    N, K = w32.shape
    b = w32.reshape(N // group, group, K)
    amax = np.max(np.abs(b), axis=(1, 2), keepdims=True)
    q, scale = q8._quantize_group_values(b, amax)
    return q.reshape(N, K), np.repeat(scale[:, 0, :].astype(np.float64), K // group, axis=1)


def _swiglu_swapped(gate, up):
    return q8.silu(up) * np.asarray(gate, np.float64)


def _add_norm_unrounded_residual(h, a, gamma, eps):
    r = np.asarray(h, np.float64) + np.asarray(a, np.float64)
    return r, np.asarray(gamma, np.float64) * r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)


def _o_proj_unrounded_a(h, o, w_o):
    a = lay.linear(o, w_o)
    return q8.round_bf16(a), q8.round_bf16(np.asarray(h, np.float64) + a)


def _ffn_gate_up_swapped(r, gamma, w_gate, w_up, w_down, eps):
    return lay.__dict__["_orig_ffn_bf16"](r, gamma, w_up, w_gate, w_down, eps)


def _final_norm_no_gamma(rows, gamma_f, eps):
    return q8.round_bf16(lay.rms_norm_rows(rows, np.ones_like(np.asarray(gamma_f, np.float64)), eps))


def _block_rows_shifted(seqs):
    return np.concatenate([np.arange(s[0] + s[2] + 1, s[0] + s[3] + 1) for s in seqs]).astype(np.int64)


def _softmax_columns(logits):
    l = np.asarray(logits, np.float64)
    e = np.exp(l - l.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def _sample_rows_last_max(hidden_rows, gamma_f, w_lm, eps):
    out = lay.__dict__["_orig_sample_rows"](hidden_rows, gamma_f, w_lm, eps)
    lg = out["logits"]
    out["token"] = lg.shape[-1] - 1 - np.argmax(lg[:, ::-1], axis=-1)
    out["confidence"] = out["probs"][np.arange(len(lg)), out["token"]]
    return out


def _approx_all_fresh(params, cfg, state, ids, seqs):
    # recomputes every row at every layer: no stale keys at all
    full = mlr.forward_full(params, cfg, ids, seqs)
    rows = np.concatenate([np.arange(o + bs, o + be) for o, _, bs, be in seqs])
    return full["X"][-1][rows]


def _approx_block_rope_from_zero(params, cfg, state, ids, seqs):
    orig = mlr.layer_qkv

    def qkv(X_rows, lp, cfg_, pos):
        return orig(X_rows, lp, cfg_, np.arange(len(pos)))
    mlr.layer_qkv = qkv
    try:
        return mlr.__dict__["_orig_approx_step"](params, cfg, state, ids, seqs)
    finally:
        mlr.layer_qkv = orig


def _schedule_refresh_off_by_one(params, cfg, ids_per_step, seqs, r):
    return mlr.__dict__["_orig_run_schedule"](params, cfg, ids_per_step, seqs, None if r is None else r + 1)


def _importance_softmax_over_queries(q_block, k, scale, n_kv_heads=None):
    q, kk = np.asarray(q_block, np.float64), np.asarray(k, np.float64)
    imp = np.zeros(kk.shape[0])
    for h in range(q.shape[1]):
        s = scale * q[:, h] @ kk[:, h * kk.shape[1] // q.shape[1]].T
        e = np.exp(s - s.max(axis=0, keepdims=True))
        imp += (e / e.sum(axis=0, keepdims=True)).sum(axis=0)
    return imp


def _tracking_ties_to_higher_row(imp, exclude, budget):
    imp = np.asarray(imp, np.float64)
    ex = set(int(x) for x in exclude)
    cand = sorted((j for j in range(len(imp)) if j not in ex), key=lambda j: (-imp[j], -j))
    return np.array(sorted(cand[:budget]), dtype=np.int64)


def _views_not_isolated(view, pos, n_ctx):
    vis = fdr.__dict__["_orig_verify_visible"](view, pos, n_ctx)
    vis[:, n_ctx:] = True
    return vis


def _accept_non_strict(draft_tok, mask_tok, mask_conf, gamma):
    n = 0
    for d, m, c in zip(draft_tok, mask_tok, mask_conf):
        if int(d) != int(m) or not float(c) >= gamma:
            break
        n += 1
    return n


MUTATIONS = {
    "rms_norm drops gamma": ("rms_norm", _rms_no_gamma),
    "rms_norm eps outside the root": ("rms_norm", _rms_eps_outside),
    "qkv_project swaps k and v": ("qkv_project", _qkv_k_v_swapped),
    "qkv_project reads heads feature-major": ("qkv_project", _qkv_heads_feature_major),
    "rope frequency theta^(-i/d)": ("rope_angles", _rope_angles_half_freq),
    "rope rotates the wrong way": ("rope", _rope_wrong_sign),
    "lse in log base 2": ("finalize", _finalize_log2),
    "online update alpha inverted": ("online_update", _online_alpha_inverted),
    "merge leaves the second state unscaled": ("merge_states", _merge_unscaled_second),
    "FACache over all keys": ("facache_canonical", _facache_all_keys),
    "grouped KV head by modulo": ("_kv_head", _kv_head_modulo),
    "attention without the scale": ("attention", _attention_unscaled),
    "cached step ropes the block from position 0": ("cached_step", _cached_step_block_at_zero),
    "fp8 rounds toward zero": ("fp8:round_e4m3", _round_e4m3_toward_zero),
    "fp8 ties away from zero": ("fp8:round_e4m3", _round_e4m3_ties_away),
    "fp8 scale amax * Q_max": ("fp8:_quantize_group_values", _quantize_group_scale_times),
    "fp8 weight scale per row stripe": ("fp8:quantize_weight", _quantize_weight_row_stripes),
    "swiglu gate and up swapped": ("fp8:swiglu", _swiglu_swapped),
    "residual not rounded to bf16": ("fp8:add_norm", _add_norm_unrounded_residual),
    "layer residual adds the unrounded projection": ("layer:o_proj_residual", _o_proj_unrounded_a),
    "layer ffn gate and up swapped": ("layer:ffn_bf16", _ffn_gate_up_swapped),
    "final norm drops gamma": ("layer:final_norm", _final_norm_no_gamma),
    "sampler cut one row late": ("layer:block_rows", _block_rows_shifted),
    "softmax over the wrong axis": ("layer:softmax_rows", _softmax_columns),
    "argmax takes the last of equal maxima": ("layer:sample_rows", _sample_rows_last_max),
    "approximate step recomputes every row": ("ml:approx_step", _approx_all_fresh),
    "approximate step ropes the block from position 0": ("ml:approx_step", _approx_block_rope_from_zero),
    "refresh interval one step late": ("ml:run_schedule", _schedule_refresh_off_by_one),
    "importance normalised over the queries": ("fd:importance", _importance_softmax_over_queries),
    "tracking ties go to the higher row": ("fd:select_tracking", _tracking_ties_to_higher_row),
    "verify views see each other": ("fd:verify_visible", _views_not_isolated),
    "acceptance threshold not strict": ("fd:verify_accept", _accept_non_strict),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mutation_fails_a_pin(mutation, monkeypatch):
    fname, fn = MUTATIONS[mutation]
    mod = ref
    if fname.startswith("fp8:"):
        mod, fname = q8, fname[4:]
    elif fname.startswith("layer:"):
        mod, fname = lay, fname[6:]
    elif fname.startswith("ml:"):
        mod, fname = mlr, fname[3:]
    elif fname.startswith("fd:"):
        mod, fname = fdr, fname[3:]
    orig = getattr(mod, fname)
    monkeypatch.setitem(mod.__dict__, f"_orig_{fname}", orig)
    monkeypatch.setattr(mod, fname, fn)
    if mod is ref and hasattr(oracle, fname):
        monkeypatch.setattr(oracle, fname, fn)
    # The mutated module's own pins first; the first failing pin settles it.
    own = {ref: pins, q8: fp8_pins, lay: layer_pins, mlr: ml_pins, fdr: fd_pins}[mod]
    calls = sorted(_pin_calls(), key=lambda c: c[1].__module__ != own.__name__)
    failed = None
    for name, pin, kwargs in calls:
        try:
            pin(**kwargs)
        except Exception:          # a wrong value, or a mutant that breaks the pin's indexing
            failed = name
            break
    print(f"{mutation}: fails {failed}")
    assert failed, f"mutation '{mutation}' passed every pin"


def test_pins_pass_without_mutation():
    for name, pin, kwargs in _pin_calls():
        pin(**kwargs)
