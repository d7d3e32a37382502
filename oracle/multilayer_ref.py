"""Plain CPU oracle of approximate deeper-layer reuse with a refresh interval.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes:
* A model of L transformer layers of one shape.  Layer l maps its input rows
  X_l to X_{l+1}: RMSNorm, the QKV projection, RoPE at each token's position
  in its sample, bidirectional softmax attention within the sample (LaCache
  Section 3.3.2 Eq. (1), Section 3.3.3), then the rest of the layer as in
  layer_ref (W_o and the residual, the feed-forward RMSNorm, SwiGLU FFN, the
  second residual).  X_0 is the embedding of the ids.
* The full recompute: every layer on every row (what a refresh computes).
* The approximate step of block-wise decoding (the DualCache page, "Block-wise
  Generation" and "Suffix Cache Refresh"; LaCache Appendix C, Figure 8):
  layer 0 exactly (LaCache's cached step equals its full recompute), and at
  every layer after the first only the block rows are recomputed: their
  fresh q, k, v attend over the layer's keys and values where every other
  row's are those of the last refresh; the other rows' inputs and outputs are
  not recomputed.  A refresh (the full recompute) happens at the first step
  of the block and every r inner steps after it (r = None: block boundary
  only).

Readings (listed in the design doc): the attention output is a bf16 tensor before
W_o (the output dtype of the cached step); the refresh rebuilds every cached
key and value of every layer; the schedule's error is measured on the block
rows of the last layer's output.  Everything else is fp64.
"""

from __future__ import annotations

import numpy as np

from . import lacache_ref as R
from .fp8_ref import round_bf16
from .layer_ref import layer0_finish

__all__ = ["layer_qkv", "layer_attention", "forward_full", "approx_step", "run_schedule"]


def layer_qkv(X_rows, lp, cfg: R.Layer0Config, pos):
    """q, k, v [n, H, d_h] (RoPE'd q and k) of input rows X_rows at positions pos."""
    q, k, v = R.qkv_project(R.rms_norm(X_rows, lp["gamma_attn"], cfg.rms_eps), lp["w_qkv"], cfg)
    return R.rope(q, pos, cfg.rope_theta), R.rope(k, pos, cfg.rope_theta), v


def layer_attention(q, k, v, cfg: R.Layer0Config):
    """O [R, H d_h] of queries q [R, H, d_h] over k, v [N, H_kv, d_h], rounded to bf16."""
    out = np.empty(q.shape)
    for h in range(cfg.n_heads):
        kh = h * cfg.n_kv_heads // cfg.n_heads
        out[:, h] = R.attention(q[:, h], k[:, kh], v[:, kh], cfg.scale)[0]
    return round_bf16(out.reshape(q.shape[0], -1))


def _finish(X_rows, O_rows, lp, eps):
    return layer0_finish(X_rows, O_rows, lp["w_o"], lp["gamma_ffn"], lp["w_gate"], lp["w_up"], lp["w_down"],
                         eps)["out"]


def forward_full(params, cfg: R.Layer0Config, ids, seqs) -> dict:
    """Every layer on every row.  Returns X [L + 1] (X[0] the embedding rows)
    and the RoPE'd k, v of every layer (the caches a refresh leaves)."""
    T = max(s[0] + s[1] for s in seqs)
    X = [R.embed(params["embed"], ids)]
    K, V = [], []
    for lp in params["layers"]:
        Xn = np.zeros_like(X[-1])
        Kl = np.zeros((T, cfg.n_kv_heads, cfg.head_dim))
        Vl = np.zeros_like(Kl)
        for off, n, _, _ in seqs:
            rows = np.arange(off, off + n)
            q, k, v = layer_qkv(X[-1][rows], lp, cfg, np.arange(n))
            Kl[rows], Vl[rows] = k, v
            Xn[rows] = _finish(X[-1][rows], layer_attention(q, k, v, cfg), lp, cfg.rms_eps)
        X.append(Xn)
        K.append(Kl)
        V.append(Vl)
    return dict(X=X, K=K, V=V)


def approx_step(params, cfg: R.Layer0Config, state, ids, seqs) -> np.ndarray:
    """One approximate inner step with the current ids, from the state of the
    last refresh (forward_full's X, K, V).  Returns the block rows of the last
    layer's output, sample by sample (block-table order)."""
    out_rows = []
    for off, n, bs, be in seqs:
        rows = np.arange(off, off + n)
        blk = np.arange(bs, be)
        # Layer 0, exactly: every row of the sample with the new ids.
        lp = params["layers"][0]
        X0 = R.embed(params["embed"], ids[rows])
        q, k, v = layer_qkv(X0, lp, cfg, np.arange(n))
        xb = _finish(X0[blk], layer_attention(q[blk], k, v, cfg), lp, cfg.rms_eps)
        # Later layers: the block rows' fresh q, k, v over the last refresh's
        # keys and values of the other rows.
        for li in range(1, len(params["layers"])):
            lp = params["layers"][li]
            qb, kb, vb = layer_qkv(xb, lp, cfg, blk)
            k = state["K"][li][rows].copy()
            v = state["V"][li][rows].copy()
            k[blk], v[blk] = kb, vb
            xb = _finish(xb, layer_attention(qb, k, v, cfg), lp, cfg.rms_eps)
        out_rows.append(xb)
    return np.concatenate(out_rows)


def run_schedule(params, cfg: R.Layer0Config, ids_per_step, seqs, r) -> dict:
    """A block's inner steps: step 0 refreshes, then step k refreshes when r
    divides k (r = None: never again) and runs the approximate step otherwise.
    Returns, per step, the block rows of the schedule's last-layer output and
    of the full recompute, and which steps refreshed."""
    rows = np.concatenate([np.arange(o + bs, o + be) for o, _, bs, be in seqs])
    got, ref, refreshed, state = [], [], [], None
    for k, ids in enumerate(ids_per_step):
        full = forward_full(params, cfg, ids, seqs)
        ref.append(full["X"][-1][rows])
        if k == 0 or (r is not None and k % r == 0):
            state = full
            got.append(full["X"][-1][rows])
            refreshed.append(True)
        else:
            got.append(approx_step(params, cfg, state, ids, seqs))
            refreshed.append(False)
    return dict(got=got, ref=ref, refreshed=refreshed, rows=rows)
