"""Attention-only parity on the GPU's own cache values.

The GPU path rounds q, k, v to fp16 when it writes the RoPECache, and the
output bar of the whole layer (2e-2) is set by that rounding: it cannot see a
key that an attention kernel drops or counts twice at a tile or segment edge.
This check takes the values the GPU itself stored (q, k, v and the FACache
triple (m, l, O~/l)), computes with the oracle's fp64 functions what the
attention over exactly those values is (LaCache Section 3.3.3, Eqs. (2)-(6):
softmax over all keys for block rows and refreshed rows; for invariant rows of
a step, the cached state updated with the block's keys), and compares every
row with bounds that only the kernels' own roundings can reach:

* LSE (fp32 output): |err| <= LSE_ATOL = 1e-4.  Score products of fp16
  operands are exact in fp32 and the sums over d_h, the exponentials and the
  normaliser carry fp32 roundings of relative size 2^-24 each, which
  accumulate to about 1e-6..1e-5 at these lengths.  A key that is dropped or
  counted twice moves the LSE of a row by about its softmax weight, 1/N on
  average (>= 2e-4 for every N <= 4864 here), and an edge bug misplaces the
  same key in every row of the tile, so rows where that key weighs more than
  average move further.
* O: |err| <= 2^-r |O_ref| + 2 (2 * 2^-p + N 2^-23) S, per element, where
  r = 8 for a bf16 output (one round-to-nearest of the result), 11 for an
  fp16 FACache entry, 24 for fp32; S = sum_j (p_j / l) |v_j| over the keys
  the kernel streamed into the accumulator (for an invariant row of a step:
  the block's keys); 2^-p (p = 11 for 16-bit caches, 24 for fp32) is the
  relative rounding of each probability before the P*V product and of the
  staging of partial outputs (two such roundings); N 2^-23 bounds the fp32
  accumulation over N keys.

The pins of this check against a planted one-key error are CPU tests
(tests/test_attn_check_cpu.py).
"""

from __future__ import annotations

import numpy as np

import oracle

LSE_ATOL = 1e-4


def o_tolerance(o_ref, s_abs, n_keys, out_bits, p_bits=11):
    """Per-element bound on |O_gpu - O_ref| (see the module docstring)."""
    return 2.0 ** -out_bits * np.abs(o_ref) + 2.0 * (2.0 * 2.0 ** -p_bits + n_keys * 2.0 ** -23) * s_abs


def _probs(q, k, scale, m, l):
    """p_j / l for rows q over keys k, given each row's final max m and normaliser l."""
    s = scale * (q @ k.T)
    return np.exp(s - m[:, None]) / l[:, None]


def full_rows(q, k, v, scale):
    """Reference O, LSE and S of rows q over every key (block rows, refreshed rows)."""
    m, l, O = oracle.state_over_keys(q, k, v, scale)
    o_ref, lse = oracle.finalize((m, l, O))
    s_abs = _probs(q, k, scale, m, l) @ np.abs(v)
    return o_ref, lse, s_abs


def invariant_rows(q_u, m_c, l_c, o_c, k_c, v_c, scale):
    """Reference O, LSE and S of invariant rows of a step: the stored FACache state
    (m_c, l_c, O~/l = o_c) updated with the block's keys k_c, v_c."""
    st = (m_c, l_c, o_c * l_c[:, None])
    m, l, O = oracle.online_update(st, q_u, k_c, v_c, scale)
    o_ref, lse = oracle.finalize((m, l, O))
    s_abs = _probs(q_u, k_c, scale, m, l) @ np.abs(v_c)
    # The cached part O~/l * (l_c e^(m_c - m) / l) is combined in fp32: a few
    # relative roundings of 2^-24 of its size.
    s_abs = s_abs + 2.0 ** -18 * np.abs(o_c * (l_c * np.exp(m_c - m) / l)[:, None])
    return o_ref, lse, s_abs


class Report:
    """Worst ratios err / bound seen (must stay <= 1)."""

    def __init__(self, p_bits=11):
        self.p_bits = p_bits
        self.worst_o = 0.0
        self.worst_lse = 0.0
        self.rows = 0

    def add(self, what, got_o, o_ref, s_abs, n_keys, out_bits, got_lse=None, lse_ref=None):
        got_o = np.asarray(got_o, np.float64)
        assert np.isfinite(got_o).all(), f"{what}: non-finite output"
        tol = o_tolerance(o_ref, s_abs, n_keys, out_bits, self.p_bits) + 1e-30
        ratio = np.abs(got_o - o_ref) / tol
        worst = float(ratio.max()) if ratio.size else 0.0
        if worst > 1.0:
            idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
            raise AssertionError(f"{what}: O error {float(np.abs(got_o - o_ref)[idx]):.3e} > bound "
                                 f"{float(tol[idx]):.3e} at {idx}")
        self.worst_o = max(self.worst_o, worst)
        if got_lse is not None:
            e = np.abs(np.asarray(got_lse, np.float64) - lse_ref)
            w = float(e.max()) if e.size else 0.0
            if w > LSE_ATOL:
                idx = int(np.argmax(e))
                raise AssertionError(f"{what}: LSE error {w:.3e} > {LSE_ATOL} at row {idx}")
            self.worst_lse = max(self.worst_lse, w)
        self.rows += len(o_ref)

    def summary(self):
        return {"rows": self.rows, "o_err_over_bound": self.worst_o, "lse_max_err": self.worst_lse}


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_sample(rep, ct, off, n, bs, be, H, Hkv, scale, kind, rows=None, heads=None, out_bits=8,
                 check_facache=True, what=""):
    """Check one sample of a cache (lacache.CacheTensors) after a refresh
    (kind "refresh": every row over every key, and the FACache snapshot of the
    invariant rows) or a block step (kind "step": block rows over every key,
    invariant rows from the stored FACache state plus the block's keys).
    rows: sample positions to check (default: all); heads: default all."""
    sl = slice(off, off + n)
    q, k, v = _f64(ct.q[sl]), _f64(ct.k[sl]), _f64(ct.v[sl])
    out, lse = _f64(ct.out[sl]), _f64(ct.lse[sl])
    rows = np.arange(n) if rows is None else np.asarray(rows)
    heads = range(H) if heads is None else heads
    in_c = (rows >= bs) & (rows < be)
    rc, ru = rows[in_c], rows[~in_c]
    Cidx = np.arange(bs, be)
    Uidx = np.r_[0:bs, be:n]
    if kind == "step":
        m_c, l_c, o_c = _f64(ct.m[sl]), _f64(ct.l[sl]), _f64(ct.o[sl])
    elif check_facache:
        m_w, l_w, o_w = _f64(ct.m[sl]), _f64(ct.l[sl]), _f64(ct.o[sl])
    for h in heads:
        kh = h // (H // Hkv)
        K, V = k[:, kh], v[:, kh]
        if kind == "refresh":
            o_ref, lse_ref, s_abs = full_rows(q[rows, h], K, V, scale)
            rep.add(f"{what} refresh h{h}", out[rows, h], o_ref, s_abs, n, out_bits, lse[rows, h], lse_ref)
            if check_facache and len(ru) and len(Uidx):
                # The snapshot: the state of invariant rows over the invariant keys only.
                m, l, O = oracle.state_over_keys(q[ru, h], K[Uidx], V[Uidx], scale)
                o_ref, pair_ref = oracle.finalize((m, l, O))
                s_abs = _probs(q[ru, h], K[Uidx], scale, m, l) @ np.abs(V[Uidx])
                rep.add(f"{what} FACache h{h}", o_w[ru, h], o_ref, s_abs, len(Uidx), min(out_bits + 3, 24),
                        m_w[ru, h] + np.log(l_w[ru, h]), pair_ref)
        else:
            if len(rc):
                o_ref, lse_ref, s_abs = full_rows(q[rc, h], K, V, scale)
                rep.add(f"{what} block rows h{h}", out[rc, h], o_ref, s_abs, n, out_bits, lse[rc, h], lse_ref)
            if len(ru):
                o_ref, lse_ref, s_abs = invariant_rows(q[ru, h], m_c[ru, h], l_c[ru, h], o_c[ru, h], K[Cidx],
                                                       V[Cidx], scale)
                rep.add(f"{what} invariant rows h{h}", out[ru, h], o_ref, s_abs, be - bs, out_bits, lse[ru, h],
                        lse_ref)
    return rep


def check_all(ct, table, cfg, kind, what="", dtype="bf16", check_facache=True):
    """Every row and head of every sample of the block table."""
    rep = Report(p_bits=11 if dtype == "bf16" else 24)
    out_bits = 8 if dtype == "bf16" else 24
    for (off, n, bs, be) in table:
        check_sample(rep, ct, off, n, bs, be, cfg.n_heads, cfg.n_kv_heads, cfg.scale, kind, out_bits=out_bits,
                     check_facache=check_facache, what=f"{what} sample@{off}")
    return rep.summary()


def check_block_query(q_block, k, v, table, out_block, lse_block, cfg, what="", dtype="bf16", samples=None,
                      heads=None):
    """DualCache block-query attention: rows of q_block over every key of their
    sample in k, v (block rows only)."""
    rep = Report(p_bits=11 if dtype == "bf16" else 24)
    out_bits = 8 if dtype == "bf16" else 24
    qb, ob, lb = _f64(q_block), _f64(out_block), _f64(lse_block)
    row0 = np.cumsum([0] + [be - bs for (_, _, bs, be) in table])
    H, Hkv = cfg.n_heads, cfg.n_kv_heads
    for b in (range(len(table)) if samples is None else samples):
        off, n, bs, be = table[b]
        K, V = _f64(k[off:off + n]), _f64(v[off:off + n])
        r = slice(row0[b], row0[b + 1])
        for h in (range(H) if heads is None else heads):
            kh = h // (H // Hkv)
            o_ref, lse_ref, s_abs = full_rows(qb[r, h], K[:, kh], V[:, kh], cfg.scale)
            rep.add(f"{what} sample {b} h{h}", ob[r, h], o_ref, s_abs, n, out_bits, lb[r, h], lse_ref)
    return rep.summary()
