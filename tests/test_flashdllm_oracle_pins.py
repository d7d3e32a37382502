"""Pins of the selective-update and verify oracle (oracle/flashdllm_ref.py).

Closed forms (importance sums to heads x queries; a dominant key takes it
all), torch's softmax and scaled_dot_product_attention with an independently
built mask, numpy's lexsort for the top-k, the view isolation as an
invariance (a draft query's output does not depend on the mask view's keys),
and the acceptance rule's closed cases.  No GPU is used.
"""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import flashdllm_ref as FD


def _rng(*s):
    return np.random.default_rng([61, *s])


def test_importance_sums_to_heads_times_queries_and_matches_torch():
    r = _rng(1)
    B, N, H, d = 7, 50, 3, 16
    q, k = r.standard_normal((B, H, d)), r.standard_normal((N, H, d))
    imp = FD.importance(q, k, 0.25)
    np.testing.assert_allclose(imp.sum(), H * B, rtol=1e-13)
    tq, tk = torch.from_numpy(q), torch.from_numpy(k)
    ref = sum(torch.softmax(0.25 * tq[:, h] @ tk[:, h].T, dim=-1).sum(0) for h in range(H)).numpy()
    np.testing.assert_allclose(imp, ref, rtol=1e-12)


def test_a_dominant_key_takes_the_importance():
    r = _rng(2)
    B, N, H, d = 4, 30, 2, 8
    u = r.standard_normal((H, d))
    q = np.repeat(u[None], B, axis=0)
    k = 0.01 * r.standard_normal((N, H, d))
    k[17] = 20.0 * u
    imp = FD.importance(q, k, 1.0)
    assert imp[17] > H * B * (1 - 1e-9) and np.argmax(imp) == 17


def test_grouped_kv_heads_share_keys():
    r = _rng(3)
    q, k = r.standard_normal((3, 4, 8)), r.standard_normal((20, 2, 8))
    imp = FD.importance(q, k, 0.5)
    k4 = np.repeat(k, 2, axis=1)                                # the same keys as 4 full heads
    np.testing.assert_allclose(imp, FD.importance(q, k4, 0.5), rtol=1e-13)


def test_select_tracking_matches_lexsort_and_breaks_ties_by_row():
    r = _rng(4)
    imp = np.round(r.random(200) * 20) / 20                    # many equal values
    exclude = np.arange(64, 96)
    got = FD.select_tracking(imp, exclude, 32)
    keep = np.setdiff1d(np.arange(200), exclude)
    order = keep[np.lexsort((keep, -imp[keep]))]
    np.testing.assert_array_equal(got, np.sort(order[:32]))
    assert len(FD.select_tracking(imp[:40], np.arange(0, 30), 32)) == 10      # fewer eligible rows


def test_visibility_rule():
    view = np.array([0, 0, 1, 1, 2, 2])
    pos = np.array([3, 5, 10, 11, 10, 11])
    vis = FD.verify_visible(view, pos, 12)
    assert not vis[:, [3, 5, 10, 11]].any() and vis[:, [0, 1, 2, 4, 6, 7, 8, 9]].all()
    own = vis[:, 12:]
    assert own[:2].tolist() == [[True, True, False, False, False, False]] * 2          # tracking: tracking only
    assert own[2:4].tolist() == [[True, True, True, True, False, False]] * 2           # draft: tracking + draft
    assert own[4:].tolist() == [[True, True, False, False, True, True]] * 2            # mask: tracking + mask


def test_verify_attention_matches_torch_sdpa_with_the_mask():
    r = _rng(5)
    N, H, d = 40, 2, 16
    view = np.array([0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2])
    pos = np.array([1, 7, 20, 30, 31, 32, 33, 30, 31, 32, 33])
    Q = len(view)
    q, kv, vv = (r.standard_normal((Q, H, d)) for _ in range(3))
    kc, vc = r.standard_normal((N, H, d)), r.standard_normal((N, H, d))
    O, L = FD.verify_attention(q, kv, vv, view, pos, kc, vc, 0.3)
    # the mask built independently: context minus carried positions, then the views
    allowed = np.ones((Q, N + Q), dtype=bool)
    allowed[:, pos] = False
    for i in range(Q):
        for j in range(Q):
            allowed[i, N + j] = (view[j] == 0) or (view[i] == view[j])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1)))
    K, V = np.concatenate([kc, kv]), np.concatenate([vc, vv])
    ref = F.scaled_dot_product_attention(t(q), t(K), t(V), attn_mask=torch.from_numpy(allowed), scale=0.3)
    np.testing.assert_allclose(O, np.swapaxes(ref.numpy(), 0, 1), rtol=1e-12, atol=1e-12)
    s = 0.3 * np.einsum("qhd,khd->hqk", q, K)
    s[:, ~allowed] = -np.inf
    np.testing.assert_allclose(L, torch.logsumexp(torch.from_numpy(s), -1).numpy().T, rtol=1e-12)


def test_views_are_isolated():
    r = _rng(6)
    N, H, d = 30, 2, 8
    view = np.array([0, 1, 1, 2, 2])
    pos = np.array([4, 20, 21, 20, 21])
    q, kv, vv = (r.standard_normal((5, H, d)) for _ in range(3))
    kc, vc = r.standard_normal((N, H, d)), r.standard_normal((N, H, d))
    O1, _ = FD.verify_attention(q, kv, vv, view, pos, kc, vc, 0.5)
    kv2, vv2 = kv.copy(), vv.copy()
    kv2[3:], vv2[3:] = 5 * r.standard_normal((2, H, d)), 5 * r.standard_normal((2, H, d))   # another mask view
    O2, _ = FD.verify_attention(q, kv2, vv2, view, pos, kc, vc, 0.5)
    np.testing.assert_array_equal(O1[:3], O2[:3])                 # tracking and draft queries unchanged
    assert np.abs(O1[3:] - O2[3:]).max() > 1e-3


def test_accept_rule_closed_cases():
    assert FD.verify_accept([5, 6, 7], [5, 6, 7], [0.9, 0.95, 0.8], 0.5) == 3
    assert FD.verify_accept([5, 6, 7], [5, 9, 7], [0.9, 0.95, 0.8], 0.5) == 1          # first mismatch stops
    assert FD.verify_accept([5, 6, 7], [5, 6, 7], [0.9, 0.5, 0.8], 0.5) == 1           # strict threshold
    assert FD.verify_accept([], [], [], 0.5) == 0
