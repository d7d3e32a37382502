"""GPU parity of the selective cache update and two-view verify
(lacache_track_select, lacache_verify_attn, lacache_verify_accept) with the
oracle (oracle/flashdllm_ref.py), on the GPU's own fp16 cache values (the
attention-only discipline of tests/attn_check.py):

* importance: against the oracle's importance of the GPU's q and k (its own
  softmax), relative 2e-3 (the GPU normalises by the attention's fp32 LSE);
  the tracking set: exactly the oracle's selection applied to the GPU's
  importance values (the decision taken in the kernel's precision), and its
  overlap with the oracle's own selection reported;
* verify attention: every row's LSE within 1e-4 and O within the bound of
  tests/attn_check.py, against the oracle's masked attention of the same
  fp16 values;
* acceptance: bit-exact counts and ids, and the order check's flag.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import flashdllm_ref as FD
from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload
import attn_check as AC

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _workloads():
    return [synth.WORKLOADS["llada8b"],
            synth.custom("fd3", prompt_lens=(200, 57, 400), gen_len=96, block_size=32, block_idx=(1, 0, 2), seed=7)]


def _stepped(wl):
    dw = DeviceWorkload(wl, device="cuda")
    dw.prefill()
    dw.block_step(dw.next_block_ids())
    torch.cuda.synchronize()
    return dw


@pytest.mark.parametrize("wi", [0, 1])
def test_track_select_matches_oracle(wi):
    wl = _workloads()[wi]
    _say(f"[track] {wl.name}: batch {wl.batch} lens {wl.seq_lens[:3]}")
    dw = _stepped(wl)
    budget = 32
    imp = torch.zeros(dw.n_rows, dtype=torch.float32, device="cuda")
    trk = torch.empty(len(dw.table), budget, dtype=torch.int32, device="cuda")
    dw.ctx.track_select(dw.ct, dw.table, budget, imp, trk)
    torch.cuda.synchronize()
    imp_g, trk_g = imp.cpu().numpy().astype(np.float64), trk.cpu().numpy()
    q = dw.ct.q.double().cpu().numpy()
    k = dw.ct.k.double().cpu().numpy()
    scale = 1.0 / np.sqrt(wl.head_dim)
    same = 0
    for b, (off, n, bs, be) in enumerate(dw.table):
        ref = FD.importance(q[off + bs:off + be], k[off:off + n], scale, wl.n_kv_heads)
        got = imp_g[off:off + n]
        np.testing.assert_allclose(got, ref, rtol=2e-3, atol=1e-6 * ref.max())
        np.testing.assert_allclose(got.sum(), wl.n_heads * (be - bs), rtol=1e-3)
        want = FD.select_tracking(got, np.arange(bs, be), budget)          # the kernel's precision
        exp = np.full(budget, -1)
        exp[:len(want)] = want
        np.testing.assert_array_equal(trk_g[b], exp)
        own = FD.select_tracking(ref, np.arange(bs, be), budget)
        same += len(set(own) & set(want))
        _say(f"  sample {b}: importance within 2e-3, tracking set = selection of the GPU's importance; "
             f"overlap with the oracle's own {len(set(own) & set(want))}/{len(own)}")
    assert same >= 0.9 * budget * len(dw.table)


def test_track_select_breaks_ties_by_row():
    """40 rows outside the block get one and the same key, aligned with the
    block queries: their importance values are bitwise equal and dominate, so
    the 32 slots are decided by the tie rule (the lower rows)."""
    wl = synth.WORKLOADS["llada8b"]
    dw = _stepped(wl)
    off, n, bs, be = dw.table[0]
    H, Hk = wl.n_heads, wl.n_kv_heads
    qm = dw.ct.q[off + bs:off + be].float().mean(0)                       # [H, d]
    kd = (qm.view(Hk, H // Hk, -1).mean(1) * 12.0).to(dw.ct.k.dtype)     # [Hk, d]
    rng = np.random.default_rng(77)
    rows = np.sort(rng.choice(np.setdiff1d(np.arange(n), np.arange(bs, be)), size=40, replace=False))
    dw.ct.k[torch.from_numpy(off + rows).cuda()] = kd
    torch.cuda.synchronize()
    budget = 32
    imp = torch.zeros(dw.n_rows, dtype=torch.float32, device="cuda")
    trk = torch.empty(len(dw.table), budget, dtype=torch.int32, device="cuda")
    dw.ctx.track_select(dw.ct, dw.table, budget, imp, trk)
    torch.cuda.synchronize()
    got = imp.cpu().numpy().astype(np.float64)[off:off + n]
    assert np.all(got[rows] == got[rows[0]]), "identical keys must get identical importance"
    assert got[rows[0]] > np.max(np.delete(got, np.concatenate([rows, np.arange(bs, be)])))
    want = FD.select_tracking(got, np.arange(bs, be), budget)
    np.testing.assert_array_equal(trk.cpu().numpy()[0], want)
    np.testing.assert_array_equal(want, rows[:budget])
    _say(f"  40 tied rows: the set is their 32 lowest rows")


@pytest.mark.parametrize("wi", [0, 1])
def test_verify_attention_matches_oracle(wi):
    wl = _workloads()[wi]
    _say(f"[verify] {wl.name}")
    dw = _stepped(wl)
    rng = np.random.default_rng([17, wi])
    H, Hk, d = wl.n_heads, wl.n_kv_heads, wl.head_dim
    views, poss, starts = [], [], [0]
    for off, n, bs, be in dw.table:
        S = min(be - bs, 24)
        others = np.setdiff1d(np.arange(n), np.arange(bs, be))
        trk = np.sort(rng.choice(others, size=min(20, len(others)), replace=False))
        search = np.arange(bs, bs + S)
        views.append(np.concatenate([np.zeros(len(trk)), np.ones(S), 2 * np.ones(S)]).astype(np.int32))
        poss.append(np.concatenate([trk, search, search]).astype(np.int32))
        starts.append(starts[-1] + len(views[-1]))
    V = starts[-1]
    view, pos = np.concatenate(views), np.concatenate(poss)
    qv = (rng.standard_normal((V, H, d)) * 2.0).astype(np.float16)
    kv = (rng.standard_normal((V, Hk, d)) * 2.0).astype(np.float16)
    vv = rng.standard_normal((V, Hk, d)).astype(np.float16)
    t = lambda x, dt=None: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = torch.empty(V, H, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(V, H, dtype=torch.float32, device="cuda")
    dw.ctx.verify_attn(t(qv), t(kv), t(vv), t(view), t(pos), starts, dw.ct, dw.table, out, lse)
    torch.cuda.synchronize()
    o_g, l_g = out.double().cpu().numpy(), lse.double().cpu().numpy()
    kc = dw.ct.k.double().cpu().numpy()
    vc = dw.ct.v.double().cpu().numpy()
    scale = 1.0 / np.sqrt(d)
    for b, (off, n, bs, be) in enumerate(dw.table):
        r = slice(starts[b], starts[b + 1])
        o_ref, l_ref = FD.verify_attention(qv[r].astype(np.float64), kv[r].astype(np.float64),
                                           vv[r].astype(np.float64), view[r], pos[r], kc[off:off + n],
                                           vc[off:off + n], scale)
        assert np.abs(l_g[r] - l_ref).max() <= AC.LSE_ATOL, np.abs(l_g[r] - l_ref).max()
        # S = sum_j p_j |v_j| over the visible keys, per query and head
        vis = FD.verify_visible(view[r], pos[r], n)
        K = np.concatenate([kc[off:off + n], kv[r].astype(np.float64)])
        Vv = np.abs(np.concatenate([vc[off:off + n], vv[r].astype(np.float64)]))
        qq = qv[r].astype(np.float64)
        for h in range(H):
            s = scale * qq[:, h] @ K[:, h * Hk // H].T
            p = np.where(vis, np.exp(s - l_ref[:, h:h + 1]), 0.0)
            s_abs = p @ Vv[:, h * Hk // H]
            tol = AC.o_tolerance(o_ref[:, h], s_abs, vis.sum(1, keepdims=True), 8)
            err = np.abs(o_g[r][:, h] - o_ref[:, h])
            assert np.all(err <= tol), f"head {h}: {err.max()} > bound"
        _say(f"  sample {b}: {starts[b + 1] - starts[b]} verify queries, LSE within {AC.LSE_ATOL}, O within the bound")


def test_verify_accept_bit_exact():
    ctx = lacache.Context(512, 4, 4, 128, 1000, 4096, 1e4, 1e-5, 0.0, "bf16")
    rng = np.random.default_rng(23)
    table = [(0, 300, 100, 164), (300, 200, 10, 42), (500, 80, 0, 16), (580, 90, 50, 82)]
    starts, draft, mtok, conf, pos, want = [0], [], [], [], [], []
    ids0 = rng.integers(0, 1000, 670).astype(np.int32)
    ids_want = ids0.copy()
    cases = [64, 20, 0, 32]                                   # search sizes (sample 2: none)
    for b, ((off, n, bs, be), S) in enumerate(zip(table, cases)):
        p = np.sort(rng.choice(np.arange(bs, be), size=S, replace=False)) if S else np.zeros(0, int)
        d = rng.integers(0, 5, S)
        m = d.copy()
        c = rng.uniform(0.6, 1.0, S)
        if b == 1:
            m[7] = (m[7] + 1) % 5                             # first mismatch at 7
        if b == 3:
            c[5] = 0.5                                        # conf == gamma at 5: not accepted
        draft.append(d); mtok.append(m); conf.append(c); pos.append(p)
        na = FD.verify_accept(d, m, c, 0.5)
        want.append(na)
        ids_want[off + p[:na]] = d[:na]
        starts.append(starts[-1] + S)
    cat = lambda xs, dt: torch.from_numpy(np.concatenate(xs).astype(dt)).cuda()
    ids = torch.from_numpy(ids0.copy()).cuda()
    nacc = torch.full((len(table),), -7, dtype=torch.int32, device="cuda")
    ctx.verify_accept(cat(draft, np.int32), cat(mtok, np.int32), cat(conf, np.float32), cat(pos, np.int32), starts,
                      table, 0.5, ids, nacc)
    torch.cuda.synchronize()
    assert nacc.cpu().tolist() == want == [64, 7, 0, 5]
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_want)
    assert ctx.read_device_status() == 0
    # positions out of order: flagged, nothing accepted in that sample
    bad = cat(pos, np.int32).clone()
    bad[[0, 1]] = bad[[1, 0]]
    ctx.verify_accept(cat(draft, np.int32), cat(mtok, np.int32), cat(conf, np.float32), bad, starts, table, 0.5,
                      ids, nacc)
    torch.cuda.synchronize()
    assert nacc[0].item() == 0 and ctx.read_device_status() & lacache.DEVFLAG_SEARCH_ORDER


def test_flashdllm_entry_points_reject_bad_arguments():
    ctx = lacache.Context(512, 4, 4, 128, 1000, 4096, 1e4, 1e-5, 0.0, "bf16")
    ct = ctx.alloc_cache(100)
    imp = torch.zeros(100, dtype=torch.float32, device="cuda")
    trk = torch.empty(1, 65, dtype=torch.int32, device="cuda")
    with pytest.raises(lacache.LaCacheError):                      # budget above 64
        ctx.track_select(ct, [(0, 100, 10, 20)], 65, imp, trk)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(lacache.LaCacheError):                      # more than 64 search positions
        ctx.verify_accept(z, z, torch.zeros(1, device="cuda"), z, [0, 65], [(0, 100, 0, 100)], 0.5, z, z)
    f32 = lacache.Context(256, 4, 4, 64, 512, 256, 1e4, 1e-5, 0.0, "f32")
    with pytest.raises(lacache.LaCacheError):                      # fp32 caches are not supported
        f32.track_select(f32.alloc_cache(100), [(0, 100, 10, 20)], 8, imp, trk[:, :8].contiguous())
