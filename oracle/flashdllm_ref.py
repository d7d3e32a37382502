"""Plain CPU oracle of Flash-dLLM's selective cache update and two-view verify.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes (the Flash-dLLM article, "Flash-Cache: Fusing Projection,
RoPE, and Cache Writes into One Kernel", its third element, and "Flash-Verify:
Making the Diffusion Model Its Own Verifier"):

* Attention importance of a sample's rows: how much softmax attention weight
  each key row receives from the current block's queries, summed over the
  queries and the heads.
* The tracking set: the `budget` decoded rows (rows outside the current
  block) of largest importance, reselected at every step.
* Two-view verify attention: a verify query holds a tracking group, the
  search positions filled with draft predictions (draft view) and the same
  positions filled with mask tokens (mask view); the views are isolated by
  the attention mask so they predict independently from shared context.
* Acceptance: a search token is accepted when the two views agree and the
  mask view's confidence exceeds gamma, sequentially in position order,
  stopping at the first failure.

Readings (listed in the design doc):
* importance_j = sum_h sum_i softmax_j(scale q_ih . k_jh) over the sample's
  keys j (every row of the sample, block rows included; they are left out of
  the selection); top-`budget` by importance, the lower row on ties;
  returned in row order.
* Views: 0 = tracking, 1 = draft, 2 = mask.  A verify query sees every
  context key (the sample's cached rows other than the positions the verify
  query itself carries), every tracking key, and the keys of its own view;
  tracking queries thus see context and tracking only.  Within a group the
  attention is bidirectional.
* Acceptance compares the views' argmax tokens; "exceeds" is strict.
Everything else is fp64.
"""

from __future__ import annotations

import numpy as np

__all__ = ["importance", "select_tracking", "verify_visible", "verify_attention", "verify_accept"]


def _softmax_rows(s):
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def importance(q_block, k, scale: float, n_kv_heads: int | None = None) -> np.ndarray:
    """Importance [N] of the key rows k [N, H_kv, d] for the block queries q_block [B, H, d]."""
    q = np.asarray(q_block, np.float64)
    k = np.asarray(k, np.float64)
    H = q.shape[1]
    Hk = k.shape[1] if n_kv_heads is None else n_kv_heads
    imp = np.zeros(k.shape[0])
    for h in range(H):
        p = _softmax_rows(scale * q[:, h] @ k[:, h * Hk // H].T)      # [B, N]
        imp += p.sum(axis=0)
    return imp


def select_tracking(imp, exclude, budget: int) -> np.ndarray:
    """The `budget` rows of largest importance outside `exclude` (lower row on
    ties), in row order; fewer when fewer rows are eligible."""
    imp = np.asarray(imp, np.float64)
    cand = [j for j in range(len(imp)) if j not in set(int(x) for x in exclude)]
    cand.sort(key=lambda j: (-imp[j], j))
    return np.array(sorted(cand[:budget]), dtype=np.int64)


def verify_visible(view, pos, n_ctx: int):
    """Boolean visibility [Q, n_ctx + Q] of the verify queries: context keys
    (columns < n_ctx, by position) except the positions the query carries,
    then the verify tokens' own keys by the view rule."""
    view = np.asarray(view)
    carried = set(int(p) for p in pos)
    ctx = np.array([j not in carried for j in range(n_ctx)])
    Q = len(view)
    vis = np.zeros((Q, n_ctx + Q), dtype=bool)
    vis[:, :n_ctx] = ctx[None, :]
    for i in range(Q):
        for j in range(Q):
            vis[i, n_ctx + j] = view[j] == 0 or view[j] == view[i]
    return vis


def verify_attention(q_ver, k_ver, v_ver, view, pos, k_ctx, v_ctx, scale: float):
    """Masked attention of the verify queries q_ver [Q, H, d] over the sample's
    context k_ctx, v_ctx [N, H_kv, d] and their own k_ver, v_ver [Q, H_kv, d].
    Returns O [Q, H, d] and LSE [Q, H] (natural log)."""
    q = np.asarray(q_ver, np.float64)
    K = np.concatenate([np.asarray(k_ctx, np.float64), np.asarray(k_ver, np.float64)])
    Vv = np.concatenate([np.asarray(v_ctx, np.float64), np.asarray(v_ver, np.float64)])
    vis = verify_visible(view, pos, np.shape(k_ctx)[0])
    Q, H, d = q.shape
    Hk = K.shape[1]
    O = np.zeros((Q, H, d))
    L = np.zeros((Q, H))
    for h in range(H):
        s = scale * q[:, h] @ K[:, h * Hk // H].T
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[:, h] = (e / l) @ Vv[:, h * Hk // H]
        L[:, h] = (m + np.log(l))[:, 0]
    return O, L


def verify_accept(draft_tok, mask_tok, mask_conf, gamma: float) -> int:
    """Number of search tokens accepted, in order: the longest prefix where the
    views agree and the mask view's confidence exceeds gamma."""
    n = 0
    for d, m, c in zip(draft_tok, mask_tok, mask_conf):
        if int(d) != int(m) or not float(c) > gamma:
            break
        n += 1
    return n
