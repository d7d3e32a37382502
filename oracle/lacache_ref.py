"""Plain fp64 CPU oracle of LaCache's exact layer-0 step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library: it receives plain NumPy arrays (already rounded to the storage dtype
by the seeded input generator) and computes everything in float64, with no
blocking, fusion or reordering beyond what the definitions below state.

What it computes (LaCache, "Exact Caching and Precision-Adaptive Inference for
Diffusion Large Language Models", arXiv 2607.16339):

* ``H = Embed(x)``, ``Hhat = Norm(H)`` (RMSNorm), ``Q,K = RoPE(Hhat W_{Q,K})``,
  ``V = Hhat W_V`` -- Section 3.3.2, Eq. (1).
* Bidirectional softmax attention of every row over every key of its own
  sequence, with the online-softmax recurrence of Section 3.3.3, Eqs. (2)-(6),
  and the log-sum-exp output of Algorithm 1 (its LSE line).
* The FACache state ``(m_cache, l_cache, O~_cache)``: the online-softmax state
  of every invariant query row restricted to the invariant keys U
  (Section 3.3.3, "FACache stores these state variables restricted to the
  unchanged region").
* The cached step: token-wise operators only for the current block C
  (EmbedCache / RoPECache, Section 3.3.2), block rows attend over all keys,
  invariant rows start from the cached state and stream only keys in C
  (Section 3.3.3, last paragraph; Figure 3 right).

Readings taken where the pages are silent (each is listed in the design doc):
softmax scale ``sm_scale`` (1/sqrt(d_h) by default; Eqs. (2) and (9) print
none), rotate-half RoPE with inverse frequency theta^(-2i/d_h) at the 0-based
position inside the sample, RMSNorm ``gamma * x / sqrt(mean(x^2) + eps)``,
grouped KV heads mapping query head ``h`` to KV head ``h // (H / H_kv)``,
FACache running max initialised to -inf (Algorithm 1 prints 0), and the cache
update of Algorithm 1 taken in the consistent form of Section 3.3.3: the cache
is its own online-softmax state over U keys.

Parity of those readings against the real LLaDA model is unpinned: the pages
fix neither the scale, the RoPE pairing nor eps.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Layer0Config", "embed", "rms_norm", "qkv_project", "rope_angles", "rope",
    "attention", "state_over_keys", "online_update", "merge_states", "finalize",
    "layer0_sample", "full_recompute", "facache_canonical", "refresh",
    "cached_step", "layer0_rows",
]


@dataclass(frozen=True)
class Layer0Config:
    """Shape and constants of the first transformer layer (Section 3.3.2)."""

    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    rope_theta: float
    rms_eps: float = 1e-5
    sm_scale: float | None = None   # None -> 1/sqrt(head_dim)

    @property
    def scale(self) -> float:
        return (1.0 / math.sqrt(self.head_dim)) if self.sm_scale is None else float(self.sm_scale)

    @property
    def n_features(self) -> int:
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim


# ----------------------------------------------------------------------------
# Token-wise operators (Section 3.3.2, Eq. (1))
# ----------------------------------------------------------------------------

def embed(E: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """H = Embed(x): the rows of the embedding table selected by the token ids."""
    return np.asarray(E[np.asarray(ids, dtype=np.int64)], dtype=np.float64)


def rms_norm(H: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Hhat = gamma * H / sqrt(mean_d H^2 + eps), one token (row) at a time."""
    H = np.asarray(H, dtype=np.float64)
    ms = np.mean(H * H, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * H / np.sqrt(ms + eps)


def qkv_project(Hhat: np.ndarray, W: np.ndarray, cfg: Layer0Config):
    """[q; k; v] = W_qkv Hhat for every token.

    ``W`` is [(H + 2 H_kv) d_h, D]: the output features of the Q heads, then the
    K heads, then the V heads, each head's ``d_h`` features contiguous.
    Returns q [T, H, d_h], k [T, H_kv, d_h], v [T, H_kv, d_h] before RoPE.
    """
    Hhat = np.asarray(Hhat, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = Hhat @ W.T
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    q = y[:, : H * d].reshape(-1, H, d)
    k = y[:, H * d: (H + Hk) * d].reshape(-1, Hk, d)
    v = y[:, (H + Hk) * d:].reshape(-1, Hk, d)
    return q, k, v


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Angle p * theta^(-2i/d_h) for every position p and pair index i < d_h/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of x [T, heads, d_h] at positions pos [T].

    Feature i is paired with feature i + d_h/2 and the pair is rotated by the
    angle of ``rope_angles``:  (a, b) -> (a cos - b sin, a sin + b cos).
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = rope_angles(pos, x.shape[-1], theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ----------------------------------------------------------------------------
# Attention and the online-softmax state (Section 3.3.3 Eqs. (2)-(6), App. B.2)
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of query rows q [R, d] over keys k, v [N, d].

    Returns O [R, d] = softmax(scale q k^T) v and LSE [R] = log sum_j exp(s_rj).
    """
    s = scale * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    O = (p @ np.asarray(v, np.float64)) / l
    return O, (m + np.log(l))[:, 0]


def state_over_keys(q, k, v, scale):
    """Online-softmax state (m, l, O~) of rows q over exactly the keys k, v.

    m = max_j s_j, l = sum_j exp(s_j - m), O~ = sum_j exp(s_j - m) v_j
    (the state of Section 3.3.3 after all listed KV blocks were streamed).
    With no keys the state is (-inf, 0, 0).
    """
    q = np.asarray(q, np.float64)
    R, d = q.shape
    if len(k) == 0:
        return np.full(R, -np.inf), np.zeros(R), np.zeros((R, np.shape(v)[-1]))
    s = scale * (q @ np.asarray(k, np.float64).T)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return m, p.sum(axis=1), p @ np.asarray(v, np.float64)


def online_update(state, q, k_tile, v_tile, scale):
    """One streamed KV block, Eqs. (2)-(6) of Section 3.3.3.

    m_new = max(m, rowmax S); alpha = exp(m - m_new); P~ = exp(S - m_new);
    l_new = alpha l + rowsum P~; O~_new = alpha O~ + P~ V.
    """
    m, l, O = state
    S = scale * (np.asarray(q, np.float64) @ np.asarray(k_tile, np.float64).T)
    m_new = np.maximum(m, S.max(axis=1))
    # exp(-inf - finite) = 0 is the intended alpha for an empty prior state.
    with np.errstate(invalid="ignore"):
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
    P = np.exp(S - m_new[:, None])
    l_new = alpha * l + P.sum(axis=1)
    O_new = alpha[:, None] * O + P @ np.asarray(v_tile, np.float64)
    return m_new, l_new, O_new


def merge_states(s1, s2):
    """Combine two online-softmax states over disjoint key sets.

    This is Eqs. (2)-(6) applied with the second state playing the role of an
    already-reduced block: m = max(m1, m2), each side rescaled by exp(m_i - m).
    """
    m1, l1, O1 = s1
    m2, l2, O2 = s2
    m = np.maximum(m1, m2)
    with np.errstate(invalid="ignore"):
        a1 = np.where(np.isneginf(m1), 0.0, np.exp(m1 - m))
        a2 = np.where(np.isneginf(m2), 0.0, np.exp(m2 - m))
    return m, a1 * l1 + a2 * l2, a1[:, None] * O1 + a2[:, None] * O2


def finalize(state):
    """O = diag(l)^-1 O~ (Section 3.3.3) and L = m + log l (Algorithm 1)."""
    m, l, O = state
    return O / l[:, None], m + np.log(l)


# ----------------------------------------------------------------------------
# Full recompute: the definition the cached step must reproduce
# ----------------------------------------------------------------------------

def _kv_head(h: int, cfg: Layer0Config) -> int:
    return h // (cfg.n_heads // cfg.n_kv_heads)


def layer0_sample(params: dict, cfg: Layer0Config, ids_b: np.ndarray) -> dict:
    """Layer-0 forward of one sequence [prompt | blocks], positions 0..N-1.

    Every row attends to every key of the same sequence (bidirectional).
    Returns h [N,D], q [N,H,d], k, v [N,H_kv,d] (after RoPE), out [N,H,d],
    lse [N,H].
    """
    ids_b = np.asarray(ids_b)
    N = len(ids_b)
    pos = np.arange(N)
    h = embed(params["embed"], ids_b)
    hhat = rms_norm(h, params["gamma"], cfg.rms_eps)
    q, k, v = qkv_project(hhat, params["w_qkv"], cfg)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    out = np.empty((N, cfg.n_heads, cfg.head_dim))
    lse = np.empty((N, cfg.n_heads))
    for hd in range(cfg.n_heads):
        kh = _kv_head(hd, cfg)
        out[:, hd], lse[:, hd] = attention(q[:, hd], k[:, kh], v[:, kh], cfg.scale)
    return dict(h=h, q=q, k=k, v=v, out=out, lse=lse)


def full_recompute(params: dict, cfg: Layer0Config, ids: np.ndarray, seqs) -> dict:
    """Layer 0 over every sample of a flat batch.

    ``ids`` [T] holds each sample's tokens at rows seq_offset .. seq_offset+N-1;
    ``seqs`` is a list of (seq_offset, seq_len, block_start, block_end).
    Rows of the flat buffers not covered by any sample are left as NaN.
    """
    ids = np.asarray(ids)
    T = len(ids)
    D, H, Hk, d = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    res = dict(h=np.full((T, D), np.nan), q=np.full((T, H, d), np.nan),
               k=np.full((T, Hk, d), np.nan), v=np.full((T, Hk, d), np.nan),
               out=np.full((T, H, d), np.nan), lse=np.full((T, H), np.nan))
    for (off, n, _bs, _be) in seqs:
        r = layer0_sample(params, cfg, ids[off:off + n])
        for key in res:
            res[key][off:off + n] = r[key]
    return res


def _split(n: int, bs: int, be: int):
    C = np.arange(bs, be)
    U = np.concatenate([np.arange(0, bs), np.arange(be, n)])
    return C, U


def facache_canonical(q, k, v, U, cfg: Layer0Config):
    """FACache of one sample: the online state of rows U over keys U.

    Returns the raw state (m, l, O~) [|U|, H], [|U|, H], [|U|, H, d] and its
    shift-free canonical pair (O~/l, m + log l).  q, k, v are one sample's
    post-RoPE rows.
    """
    H, d = cfg.n_heads, cfg.head_dim
    m = np.empty((len(U), H)); l = np.empty((len(U), H)); O = np.empty((len(U), H, d))
    for hd in range(H):
        kh = _kv_head(hd, cfg)
        m[:, hd], l[:, hd], O[:, hd] = state_over_keys(q[U, hd], k[U, kh], v[U, kh], cfg.scale)
    return (m, l, O), (O / l[..., None], m + np.log(l))


def refresh(params: dict, cfg: Layer0Config, ids: np.ndarray, seqs) -> dict:
    """First denoising step of a block: full recompute plus the caches.

    Adds ``m_c``, ``l_c``, ``o_c`` (FACache state, rows of U only; C rows NaN)
    to the result of ``full_recompute``: Section 3.3 ("populated at the first
    denoising step of each SAR block").
    """
    res = full_recompute(params, cfg, ids, seqs)
    T = len(ids)
    H, d = cfg.n_heads, cfg.head_dim
    res["m_c"] = np.full((T, H), np.nan)
    res["l_c"] = np.full((T, H), np.nan)
    res["o_c"] = np.full((T, H, d), np.nan)
    for (off, n, bs, be) in seqs:
        _, U = _split(n, bs, be)
        if len(U) == 0:
            continue
        sl = slice(off, off + n)
        (m, l, O), _ = facache_canonical(res["q"][sl], res["k"][sl], res["v"][sl], U, cfg)
        res["m_c"][off + U] = m
        res["l_c"][off + U] = l
        res["o_c"][off + U] = O
    return res


def cached_step(params: dict, cfg: Layer0Config, cache: dict, block_ids: np.ndarray,
                seqs, kv_tile: int = 16) -> dict:
    """The cached inner step, plainly, in fp64 (Section 3.3.2-3.3.3).

    ``cache`` holds h, q, k, v (all rows, from the refresh) and the FACache
    state m_c, l_c, o_c of the invariant rows.  ``block_ids`` [sum B_b] are the
    current block's ids, concatenated in sample order.  Only block rows go
    through the token-wise operators; block rows attend over all keys; every
    invariant row starts from its cached state and streams only the block's
    keys, ``kv_tile`` keys at a time, with Eqs. (2)-(6).  Returns new h, q, k,
    v (copies, block rows replaced), out and lse for all rows.  The FACache is
    not modified (Algorithm 1 stores it only at the first step).
    """
    H, Hk, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    h = cache["h"].copy(); q = cache["q"].copy(); k = cache["k"].copy(); v = cache["v"].copy()
    T = h.shape[0]
    out = np.full((T, H, d), np.nan)
    lse = np.full((T, H), np.nan)
    block_ids = np.asarray(block_ids)
    cur = 0
    for (off, n, bs, be) in seqs:
        B = be - bs
        rows = off + np.arange(bs, be)
        # EmbedCache / RoPECache: recompute the token-wise operators for C only.
        hc = embed(params["embed"], block_ids[cur:cur + B])
        cur += B
        qc, kc, vc = qkv_project(rms_norm(hc, params["gamma"], cfg.rms_eps), params["w_qkv"], cfg)
        pos = np.arange(bs, be)
        h[rows] = hc
        q[rows] = rope(qc, pos, cfg.rope_theta)
        k[rows] = rope(kc, pos, cfg.rope_theta)
        v[rows] = vc
        C, U = _split(n, bs, be)
        for hd in range(H):
            kh = _kv_head(hd, cfg)
            ks, vs = k[off:off + n, kh], v[off:off + n, kh]
            # Query rows inside C: stream every KV block.
            out[off + C, hd], lse[off + C, hd] = attention(q[off + C, hd], ks, vs, cfg.scale)
            if len(U) == 0:
                continue
            # Query rows inside U: initialise from FACache, stream KV blocks of C.
            st = (cache["m_c"][off + U, hd].copy(), cache["l_c"][off + U, hd].copy(),
                  cache["o_c"][off + U, hd].copy())
            for j0 in range(bs, be, kv_tile):
                j1 = min(be, j0 + kv_tile)
                st = online_update(st, q[off + U, hd], ks[j0:j1], vs[j0:j1], cfg.scale)
            out[off + U, hd], lse[off + U, hd] = finalize(st)
    return dict(h=h, q=q, k=k, v=v, out=out, lse=lse)


def layer0_rows(params: dict, cfg: Layer0Config, ids_b: np.ndarray, rows, heads) -> dict:
    """Layer-0 output of selected rows and heads of one sequence.

    The same definition as ``layer0_sample`` restricted to what the selected
    outputs depend on: q of the selected rows, k and v of every row, for the
    selected heads only.  Used to check large workloads on sampled outputs.
    Returns out [len(rows), len(heads), d] and lse [len(rows), len(heads)].
    """
    ids_b = np.asarray(ids_b)
    rows = np.asarray(rows)
    N = len(ids_b)
    d, H, Hk = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
    h = embed(params["embed"], ids_b)
    hhat = rms_norm(h, params["gamma"], cfg.rms_eps)
    W = params["w_qkv"]
    out = np.empty((len(rows), len(heads), d))
    lse = np.empty((len(rows), len(heads)))
    pos = np.arange(N)
    for j, hd in enumerate(heads):
        kh = _kv_head(hd, cfg)
        wq = np.asarray(W[hd * d:(hd + 1) * d], np.float64)
        wk = np.asarray(W[(H + kh) * d:(H + kh + 1) * d], np.float64)
        wv = np.asarray(W[(H + Hk + kh) * d:(H + Hk + kh + 1) * d], np.float64)
        qh = rope((hhat[rows] @ wq.T)[:, None, :], pos[rows], cfg.rope_theta)[:, 0]
        kh_ = rope((hhat @ wk.T)[:, None, :], pos, cfg.rope_theta)[:, 0]
        vh = hhat @ wv.T
        out[:, j], lse[:, j] = attention(qh, kh_, vh, cfg.scale)
    return dict(out=out, lse=lse)
