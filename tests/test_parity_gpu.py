"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case prints its name, shapes and seed before touching the GPU.  Small
workloads are compared element by element on every row; the full-size
workloads are compared on sampled (sample, row, head) outputs that the
oracle computes one by one.
"""

import sys

import numpy as np
import pytest
import torch

import attn_check
import oracle
from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload
from helpers import cfg_of, check_cache_values, check_lse, check_output, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _facache_pair(dw, rows):
    m, l, o = host(dw.ct.m)[rows], host(dw.ct.l)[rows], host(dw.ct.o)[rows]
    return o, m + np.log(l)


def _compare_refresh(dw, ref, what):
    wl = dw.wl
    rows = np.concatenate([np.arange(off, off + n) for (off, n, _, _) in dw.table])
    assert np.array_equal(host(dw.ct.h)[rows], ref["h"][rows]), f"{what}: EmbedCache rows differ from the table"
    for key in ("q", "k", "v"):
        check_cache_values(host(getattr(dw.ct, key))[rows], ref[key][rows], wl.dtype, f"{what} {key}")
    stats = check_output(host(dw.ct.out)[rows], ref["out"][rows], wl.dtype, f"{what} out")
    check_lse(host(dw.ct.lse)[rows], ref["lse"][rows], wl.dtype, f"{what} lse")
    urows = np.concatenate([off + np.r_[0:bs, be:n] for (off, n, bs, be) in dw.table])
    if len(urows):
        o_pair, lse_pair = _facache_pair(dw, urows)
        ref_o = ref["o_c"][urows] / ref["l_c"][urows][..., None]
        ref_lse = ref["m_c"][urows] + np.log(ref["l_c"][urows])
        check_output(o_pair, ref_o, wl.dtype, f"{what} FACache O~/l")
        check_lse(lse_pair, ref_lse, wl.dtype, f"{what} FACache m+ln l")
    return stats


def _compare_step(dw, ref, what):
    wl = dw.wl
    rows = np.concatenate([np.arange(off, off + n) for (off, n, _, _) in dw.table])
    crow = np.concatenate([off + np.arange(bs, be) for (off, n, bs, be) in dw.table])
    assert np.array_equal(host(dw.ct.h)[crow], ref["h"][crow]), f"{what}: EmbedCache block rows"
    for key in ("q", "k", "v"):
        check_cache_values(host(getattr(dw.ct, key))[crow], ref[key][crow], wl.dtype, f"{what} {key}")
    stats = check_output(host(dw.ct.out)[rows], ref["out"][rows], wl.dtype, f"{what} out")
    check_lse(host(dw.ct.lse)[rows], ref["lse"][rows], wl.dtype, f"{what} lse")
    return stats


def _run_full(wl, steps, packed=True, dw=None):
    """Refresh, then `steps` inner steps, every row against the oracle (the
    layer's output bar) and against the attention over the GPU's own cache
    values (tests/attn_check.py); the device status word must stay clear (no
    fp16 range overflow, no bad id)."""
    _say(f"[parity] {wl.name}: dtype {wl.dtype} D {wl.d_model} H {wl.n_heads}x{wl.head_dim} "
         f"batch {wl.batch} seq_lens {wl.seq_lens[:4]}... block {wl.block_size} seed {wl.seed} packed {packed}")
    dw = dw or DeviceWorkload(wl, packed=packed)
    cfg = cfg_of(wl)
    dw.prefill()
    torch.cuda.synchronize()
    ref = oracle.refresh(dw.params, cfg, dw.ids_host, dw.table)
    st = _compare_refresh(dw, ref, f"{wl.name} refresh")
    at = attn_check.check_all(dw.ct, dw.table, cfg, "refresh", f"{wl.name} refresh", wl.dtype)
    _say(f"[parity] {wl.name} refresh ok {st} attention-only {at}")
    for s in range(1, steps + 1):
        blk = dw.next_block_ids()
        dw.block_step(blk)
        torch.cuda.synchronize()
        ref = oracle.full_recompute(dw.params, cfg, dw.ids_host, dw.table)
        st = _compare_step(dw, ref, f"{wl.name} step {s}")
        at = attn_check.check_all(dw.ct, dw.table, cfg, "step", f"{wl.name} step {s}", wl.dtype)
        _say(f"[parity] {wl.name} step {s} ok {st} attention-only {at}")
    flags = dw.ctx.read_device_status()
    assert flags == 0, f"{wl.name}: device status flags {flags:#x} after the run"
    return dw


def test_tiny_fp32_refresh_and_steps():
    _run_full(synth.WORKLOADS["tiny"], 3)


@pytest.mark.parametrize("packed", [True, False])
def test_small_bf16_ragged_batch(packed):
    # Three samples: ragged lengths (not multiples of any tile), a block at the
    # very start, a block at the very end, and grouped KV heads.  42 block
    # tokens: the skinny packed-weight GEMM (packed) or the streaming
    # small-batch kernel.
    wl = synth.custom("small_bf16_ragged", dtype="bf16", d_model=512, n_heads=4, n_kv_heads=2, head_dim=128,
                      vocab=3000, prompt_lens=(37, 150, 5), gen_len=70, block_size=14, block_idx=(2, 0, 4),
                      steps=3, seed=21)
    _run_full(wl, 3, packed=packed)


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_refresh_segment_edges(head_dim, rows, monkeypatch):
    # The refresh streams the invariant keys in two segments, then the block's
    # keys, each segment in 64-key tiles: a block at position 0 (empty first
    # segment), blocks at the very end (empty second segment), a 40-key block
    # (ragged block tile), and a sample spanning four 128-row items (420 rows);
    # grouped KV heads.  Every row and every FACache pair is compared, with
    # 64-row and 128-row refresh workgroups (fixed through LACACHE_REFRESH_ROWS).
    monkeypatch.setenv("LACACHE_REFRESH_ROWS", str(rows))
    wl = synth.custom(f"refresh_edges_h{head_dim}", dtype="bf16", d_model=512, n_heads=4, n_kv_heads=2,
                      head_dim=head_dim, vocab=1200, prompt_lens=(0, 130, 61, 300), gen_len=120, block_size=40,
                      block_idx=(0, 2, 2, 1), steps=1, seed=51)
    _run_full(wl, 1)


def test_refresh_rows_per_workgroup_bitwise(monkeypatch):
    """The rows per refresh workgroup (64 or 128) change no row's arithmetic:
    both launches give bit-identical outputs, LSE and FACache."""
    wl = synth.custom("refresh_rows", dtype="bf16", d_model=512, n_heads=4, head_dim=128, vocab=900,
                      prompt_lens=(100, 7, 250), gen_len=64, block_size=32, block_idx=(1, 0, 1), steps=1, seed=53)
    res = {}
    for rows in (64, 128):
        monkeypatch.setenv("LACACHE_REFRESH_ROWS", str(rows))
        dw = DeviceWorkload(wl)
        dw.prefill()
        torch.cuda.synchronize()
        res[rows] = {k: getattr(dw.ct, k).clone() for k in ("out", "lse", "m", "l", "o")}
    urows = torch.from_numpy(np.concatenate([off + np.r_[0:bs, be:n] for (off, n, bs, be) in wl.table()])).to("cuda")
    for k in ("out", "lse"):
        assert torch.equal(res[64][k], res[128][k]), k
    for k in ("m", "l", "o"):
        assert torch.equal(res[64][k].index_select(0, urows), res[128][k].index_select(0, urows)), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_boundary_refresh(dtype):
    # At a block boundary the finished block's ids change (its final ids) and
    # the block table moves to the next block.  lacache_refresh_block
    # re-projects only the finished block's rows and recomputes the attention
    # with the new table; the result must equal the oracle's refresh of the new
    # ids on the new table (every row, every cache entry, every FACache pair).
    d_model, head_dim = (512, 128) if dtype == "bf16" else (256, 64)
    wl = synth.custom(f"block_refresh_{dtype}", dtype=dtype, d_model=d_model, n_heads=4, n_kv_heads=2,
                      head_dim=head_dim, vocab=1500, prompt_lens=(37, 100, 0), gen_len=96, block_size=32,
                      block_idx=(0, 1, 1), steps=1, seed=71)
    _say(f"[parity] {wl.name}: table {wl.table()}")
    dw = DeviceWorkload(wl)
    cfg = cfg_of(wl)
    dw.prefill()
    rng = np.random.default_rng([20261202, 71])
    ids_new = np.array(dw.ids_host, copy=True)
    proj = dw.table
    for (off, n, bs, be) in proj:
        ids_new[off + bs:off + be] = rng.integers(0, wl.vocab, size=be - bs)
    proj_ids = np.concatenate([ids_new[off + bs:off + be] for (off, n, bs, be) in proj]).astype(np.int32)
    new_table = [(off, n, be, be + (be - bs)) for (off, n, bs, be) in proj]
    ws = dw.ctx.alloc_workspace(lacache.OP_REFRESH_BLOCK, proj)
    dw.ctx.refresh_block(dw.weights, torch.from_numpy(proj_ids).cuda(), proj, new_table, dw.ct, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.refresh(dw.params, cfg, ids_new, new_table)
    dw.table = new_table
    st = _compare_refresh(dw, ref, f"{wl.name} block refresh")
    _say(f"[parity] {wl.name} block refresh ok {st}")


def test_batch_beyond_one_launch_slice():
    # 70 samples: the library launches at most 64 samples' block table per
    # kernel, so the refresh and every step run as two slices (64 + 6) with
    # different kernel paths (the first slice has enough items for the
    # whole-sequence streaming block-row kernel, the second does not).
    # Ragged prompt lengths 0..40, blocks of 16, random block positions.
    rng = np.random.default_rng([20261202, 70])
    prompts = tuple(int(x) for x in rng.integers(0, 41, size=70))
    wl = synth.custom("batch70", dtype="bf16", d_model=512, n_heads=4, head_dim=128, vocab=900,
                      prompt_lens=prompts, gen_len=32, block_size=16, steps=2, seed=61)
    _run_full(wl, 2)


@pytest.mark.parametrize("lengths", ["equal", "ragged"])
def test_streaming_kernels_head64_every_row(lengths):
    """A batch large enough for the streaming block-row kernel (whole-sequence
    chunks: 16 samples x 16 heads = 256 items) and the streaming invariant-row
    kernel (more than 2048 (64-row tile, head) items) at head_dim 64, every row
    against the oracle.  equal: every sample's invariant rows split into equal
    segments; ragged: 128-row segments."""
    if lengths == "equal":
        prompts = (600,) * 16
    else:
        rng = np.random.default_rng([20261202, 72])
        prompts = tuple(int(x) for x in rng.integers(500, 701, size=16))
    wl = synth.custom(f"stream_h64_{lengths}", dtype="bf16", d_model=1024, n_heads=16, head_dim=64, vocab=3000,
                      prompt_lens=prompts, gen_len=64, block_size=32, steps=1, seed=72)
    _run_full(wl, 1)


def test_small_fp32_head64_multi_tile():
    wl = synth.custom("small_fp32_h64", dtype="f32", d_model=256, n_heads=4, head_dim=64, vocab=700,
                      prompt_lens=(300, 77), gen_len=96, block_size=32, block_idx=(1, 2), steps=2,
                      embed_std=0.02, seed=22)
    _run_full(wl, 2)


@pytest.mark.parametrize("packed,tile", [(True, None), (True, "whole"), (True, "half"), (True, "wide"),
                                         (False, None)])
@pytest.mark.parametrize("shape", ["h128_gqa", "h64"])
def test_many_token_projection_every_row(shape, packed, tile, monkeypatch):
    """Block steps of >= 128 tokens run the MFMA GEMM projection (and so does
    every refresh): both weight forms, every row against the oracle, and each
    tile of the packed-weight GEMM (chosen by launch size, or fixed through
    LACACHE_GEMM_TILE): 128 x 192, 128 x 96 and 256 x 192.  h128_gqa:
    F = 2048 is not a multiple of the 192-column tile (a partial last tile,
    and an empty last half-width tile) and K/V head boundaries fall inside
    tiles; 320 block tokens are 2.5 row tiles (1.25 wide ones: the second
    row tile of the last wide tile lies past the launch)."""
    if tile is not None:
        monkeypatch.setenv("LACACHE_GEMM_TILE", tile)
    if shape == "h128_gqa":
        wl = synth.custom("gemm_h128_gqa", dtype="bf16", d_model=1024, n_heads=8, n_kv_heads=4, head_dim=128,
                          vocab=2000, prompt_lens=(40, 7, 96, 130, 3, 64, 21, 50, 77, 12), gen_len=64,
                          block_size=32, block_idx=(0, 1, 1, 0, 1, 0, 1, 0, 1, 1), steps=2, seed=41)
    else:
        wl = synth.custom("gemm_h64", dtype="bf16", d_model=512, n_heads=8, head_dim=64, vocab=1500,
                          prompt_lens=(20, 33, 48, 9, 60, 17, 40, 28), gen_len=32, block_size=16,
                          block_idx=(0, 1, 1, 0, 0, 1, 0, 1), steps=2, seed=42)
    assert wl.block_tokens >= 128
    _say(f"[parity] GEMM tile {tile or 'by launch size'}")
    _run_full(wl, 2, packed=packed)


def test_tiny_batched16_fp32():
    _run_full(synth.WORKLOADS["tiny_batched16"], 2)


def test_llada8b_config_all_steps():
    """Batch 1, N 768, block 32 at [608, 640): refresh + all 20 inner steps, every row."""
    _run_full(synth.WORKLOADS["llada8b"], 20)


def test_dualcache_attention_equals_block_rows_of_full_recompute():
    wl = synth.custom("dualcache_small", dtype="bf16", d_model=512, n_heads=4, head_dim=128, vocab=2000,
                      prompt_lens=(200, 31, 600), gen_len=64, block_size=32, block_idx=(1, 0, 1), seed=23)
    _say(f"[parity] dualcache on {wl.name}")
    dw = DeviceWorkload(wl)
    dw.prefill()
    crow = np.concatenate([off + np.arange(bs, be) for (off, n, bs, be) in dw.table])
    crow_t = torch.from_numpy(crow).to("cuda")
    q_block = dw.ct.q.index_select(0, crow_t).contiguous()
    out_block = torch.empty(q_block.shape, dtype=dw.ctx.torch_dtype, device="cuda")
    lse_block = torch.empty(q_block.shape[:2], dtype=torch.float32, device="cuda")
    ws = dw.ctx.alloc_workspace(lacache.OP_DUALCACHE_ATTN, dw.table)
    dw.ctx.dualcache_attn(q_block, dw.ct.k, dw.ct.v, dw.table, out_block, lse_block, ws)
    torch.cuda.synchronize()
    ref = oracle.full_recompute(dw.params, cfg_of(wl), dw.ids_host, dw.table)
    check_output(host(out_block), ref["out"][crow], wl.dtype, "dualcache out")
    check_lse(host(lse_block), ref["lse"][crow], wl.dtype, "dualcache lse")


# ---------------------------------------------------------------------------
# Full-size workloads: sampled outputs, each computed by the oracle one by one
# ---------------------------------------------------------------------------

def _sample_rows(rng, n, bs, be, k):
    """Block rows, their neighbours, both ends, and random invariant rows."""
    fixed = [0, max(bs - 1, 0), bs, (bs + be) // 2, be - 1, min(be, n - 1), n - 1]
    rand = rng.choice(n, size=min(k, n), replace=False).tolist()
    return sorted(set(int(r) for r in fixed + rand if 0 <= r < n))


def _check_sampled(dw, rng, n_samples, heads, what, k_rows=12, kind="step", tight_rows=64):
    """Sampled (sample, row, head) outputs against the oracle's layer0_rows; on
    the same samples, `tight_rows` random rows (plus the block's edges) against
    the attention over the GPU's own cache values."""
    wl = dw.wl
    cfg = cfg_of(wl)
    samples = rng.choice(len(dw.table), size=min(n_samples, len(dw.table)), replace=False)
    worst = {}
    rep = attn_check.Report()
    for b in samples:
        off, n, bs, be = dw.table[b]
        rows = _sample_rows(rng, n, bs, be, k_rows)
        ref = oracle.layer0_rows(dw.params, cfg, dw.ids_host[off:off + n], rows, heads)
        idx = torch.from_numpy(off + np.asarray(rows)).to(dw.ct.out.device)
        got_o = host(dw.ct.out.index_select(0, idx))[:, heads]
        got_l = host(dw.ct.lse.index_select(0, idx))[:, heads]
        st = check_output(got_o, ref["out"], wl.dtype, f"{what} sample {b}")
        check_lse(got_l, ref["lse"], wl.dtype, f"{what} sample {b}")
        worst = {k: max(worst.get(k, 0.0), v) for k, v in st.items()}
        trows = sorted(set(_sample_rows(rng, n, bs, be, tight_rows)) | {bs, be - 1})
        attn_check.check_sample(rep, dw.ct, off, n, bs, be, cfg.n_heads, cfg.n_kv_heads, cfg.scale, kind,
                                rows=trows, heads=heads, what=f"{what} sample {b}")
    worst["attention_only"] = rep.summary()
    return worst


@pytest.mark.parametrize("name", ["batched16", "long4", "varlen32"])
def test_full_size_configs_sampled(name):
    """Refresh, step 1 and step 20 at full size; sampled rows/heads vs the oracle."""
    wl = synth.WORKLOADS[name]
    _say(f"[parity] {name}: batch {wl.batch} seq_lens {wl.seq_lens[:6]}... block {wl.block_size} "
         f"T {wl.total_tokens} M {wl.block_tokens}")
    rng = np.random.default_rng([11, len(name)])
    heads = [0, 7, 31]
    dw = DeviceWorkload(wl)
    dw.prefill()
    torch.cuda.synchronize()
    _say(f"[parity] {name} refresh {_check_sampled(dw, rng, 3, heads, name + ' refresh', kind='refresh')}")
    for s in range(1, wl.steps + 1):
        blk = dw.next_block_ids()
        dw.block_step(blk)
        if s in (1, wl.steps):
            torch.cuda.synchronize()
            _say(f"[parity] {name} step {s} {_check_sampled(dw, rng, 3, heads, f'{name} step {s}')}")
    assert dw.ctx.read_device_status() == 0


def _dualcache_sampled(dw, rng, heads, what, n_samples=4):
    """DualCache block-query attention over the current caches: sampled samples
    against the oracle (every block row, `heads`) and against the attention over
    the GPU's own q/k/v values."""
    wl = dw.wl
    cfg = cfg_of(wl)
    crow = np.concatenate([off + np.arange(bs, be) for (off, n, bs, be) in dw.table])
    q_block = dw.ct.q.index_select(0, torch.from_numpy(crow).to("cuda")).contiguous()
    out_block = torch.empty(q_block.shape, dtype=dw.ctx.torch_dtype, device="cuda")
    lse_block = torch.empty(q_block.shape[:2], dtype=torch.float32, device="cuda")
    ws = dw.ctx.alloc_workspace(lacache.OP_DUALCACHE_ATTN, dw.table)
    dw.ctx.dualcache_attn(q_block, dw.ct.k, dw.ct.v, dw.table, out_block, lse_block, ws)
    torch.cuda.synchronize()
    got_o, got_l = host(out_block), host(lse_block)
    row0 = np.cumsum([0] + [be - bs for (_, _, bs, be) in dw.table])
    samples = rng.choice(len(dw.table), size=n_samples, replace=False)
    for b in samples:
        off, n, bs, be = dw.table[b]
        ref = oracle.layer0_rows(dw.params, cfg, dw.ids_host[off:off + n], list(range(bs, be)), heads)
        sl = slice(row0[b], row0[b + 1])
        check_output(got_o[sl][:, heads], ref["out"], wl.dtype, f"{what} sample {b}")
        check_lse(got_l[sl][:, heads], ref["lse"], wl.dtype, f"{what} sample {b}")
    at = attn_check.check_block_query(q_block, dw.ct.k, dw.ct.v, dw.table, out_block, lse_block, cfg, what,
                                      wl.dtype, samples=samples)
    _say(f"[parity] {what}: samples {sorted(int(x) for x in samples)} ok, attention-only {at}")


def test_varlen32_dualcache_attention_sampled():
    """DualCache block-query attention on the variable-length batch (block rows
    only) after the refresh, after step 1 and after step 20: the caches the
    DualCache reads are the block step's, so its output must equal the oracle
    on the current ids."""
    wl = synth.WORKLOADS["varlen32"]
    _say(f"[parity] varlen32 dualcache: batch {wl.batch}")
    dw = DeviceWorkload(wl)
    dw.prefill()
    rng = np.random.default_rng(5)
    heads = [1, 16, 30]
    _dualcache_sampled(dw, rng, heads, "varlen32 dualcache after refresh")
    for s in range(1, wl.steps + 1):
        dw.block_step(dw.next_block_ids())
        if s in (1, wl.steps):
            _dualcache_sampled(dw, rng, heads, f"varlen32 dualcache after step {s}")
    assert dw.ctx.read_device_status() == 0


def test_varlen32_batched_equals_per_sample_within_tolerance():
    """Each sample of the variable-length batch alone (its own launches, hence
    its own kernel paths and key chunks) against the same sample inside the
    32-sample batch, after the refresh and one step: equal within the output
    bar (the key chunks follow the launch's size, so the two can round
    differently; identical launches are bitwise equal, tested on small
    batches)."""
    wl = synth.WORKLOADS["varlen32"]
    _say(f"[parity] varlen32 batched vs alone: batch {wl.batch}")
    dw = DeviceWorkload(wl)
    dw.prefill()
    blk = dw.next_block_ids()
    dw.block_step(blk)
    torch.cuda.synchronize()
    worst = {}
    crow0 = 0
    # One more cache over the same weights; each sample alone runs in it.
    one = DeviceWorkload.__new__(DeviceWorkload)
    one.__dict__.update(dw.__dict__)
    one.ct = dw.ctx.alloc_cache(dw.n_rows)
    for b, (off, n, bs, be) in enumerate(dw.table):
        B = be - bs
        one.table = [(off, n, bs, be)]
        one.ids_host = synth.initial_ids(wl)
        one.prefill()
        one.ctx.block_step(one.weights, blk[crow0:crow0 + B].contiguous(), one.table, one.ct,
                           one.ctx.alloc_workspace(lacache.OP_BLOCK_STEP, one.table))
        torch.cuda.synchronize()
        rows = slice(off, off + n)
        st = check_output(host(one.ct.out[rows]), host(dw.ct.out[rows]), wl.dtype, f"sample {b} out")
        check_lse(host(one.ct.lse[rows]), host(dw.ct.lse[rows]), wl.dtype, f"sample {b} lse")
        worst = {k: max(worst.get(k, 0.0), v) for k, v in st.items()}
        crow0 += B
    _say(f"[parity] varlen32 batched vs alone ok, worst {worst}")


# ---------------------------------------------------------------------------
# Bit-exact indexing, determinism and edge cases
# ---------------------------------------------------------------------------

def _small_batched(seed=31, dtype="bf16"):
    return synth.custom("bitexact", dtype=dtype, d_model=512, n_heads=4, n_kv_heads=2, head_dim=128, vocab=900,
                        prompt_lens=(33, 170, 64, 7), gen_len=64, block_size=16, block_idx=(1, 3, 0, 2), steps=2,
                        seed=seed)


def test_batched_equals_per_sample_bitwise():
    """A sample's results do not depend on the other samples of the batch."""
    wl = _small_batched()
    _say(f"[bitexact] batched vs per-sample on {wl.name}")
    dw = DeviceWorkload(wl)
    dw.prefill()
    blk = dw.next_block_ids()
    dw.block_step(blk)
    torch.cuda.synchronize()
    full = {k: getattr(dw.ct, k).clone() for k in ("h", "q", "k", "v", "out", "lse", "m", "l", "o")}
    crow0 = 0
    for b, (off, n, bs, be) in enumerate(dw.table):
        B = be - bs
        one = DeviceWorkload(wl, ctx=dw.ctx, n_rows=dw.n_rows)
        one.table = [(off, n, bs, be)]
        one.ids_host = synth.initial_ids(wl)
        one.prefill()
        one.ctx.block_step(one.weights, blk[crow0:crow0 + B].contiguous(), one.table, one.ct,
                           one.ctx.alloc_workspace(lacache.OP_BLOCK_STEP, one.table))
        torch.cuda.synchronize()
        rows = slice(off, off + n)
        for k in ("h", "q", "k", "v", "out", "lse"):
            assert torch.equal(getattr(one.ct, k)[rows], full[k][rows]), f"sample {b}: {k} differs"
        urows = torch.from_numpy(off + np.r_[0:bs, be:n]).to("cuda")
        for k in ("m", "l", "o"):
            assert torch.equal(getattr(one.ct, k).index_select(0, urows), full[k].index_select(0, urows)), k
        crow0 += B


def test_repeated_step_is_bitwise_deterministic():
    wl = _small_batched(seed=32)
    dw = DeviceWorkload(wl)
    dw.prefill()
    blk = dw.next_block_ids()
    dw.block_step(blk)
    torch.cuda.synchronize()
    first = (dw.ct.out.clone(), dw.ct.lse.clone(), dw.ct.q.clone())
    for _ in range(3):
        dw.block_step(blk)
    torch.cuda.synchronize()
    assert torch.equal(first[0], dw.ct.out) and torch.equal(first[1], dw.ct.lse) and torch.equal(first[2], dw.ct.q)


def test_rows_outside_the_block_table_are_untouched():
    """Sentinel-filled rows that belong to no sample keep their bytes; a block step
    rewrites only the block rows of the caches and never the FACache."""
    wl = synth.custom("sentinel", dtype="bf16", d_model=512, n_heads=4, head_dim=128, vocab=500,
                      prompt_lens=(40, 50), gen_len=32, block_size=16, block_idx=(1, 0), seed=33)
    ctx = lacache.context_for(wl)
    gap = 17
    table = [(3, 72, 56, 72), (3 + 72 + gap, 82, 50, 66)]
    n_rows = table[-1][0] + table[-1][1] + 9
    dw = DeviceWorkload(wl, ctx=ctx, n_rows=n_rows)
    dw.table = table
    ids = np.zeros(n_rows, np.int32)
    base = synth.initial_ids(wl)
    ids[3:75] = base[:72]
    ids[92:174] = base[72:154]
    for t in dw.ct.__dict__.values():
        if t.dtype in (torch.float32, torch.float16, torch.bfloat16):
            t.fill_(-1024.0)
    dw.ctx.prefill_cache(dw.weights, torch.from_numpy(ids).cuda(), table, dw.ct,
                         workspace=dw.ctx.alloc_workspace(lacache.OP_PREFILL, table))
    torch.cuda.synchronize()
    outside = np.r_[0:3, 75:92, 174:n_rows]
    for k in ("h", "q", "k", "v", "out", "lse", "m", "l", "o"):
        t = getattr(dw.ct, k).float().cpu().numpy()
        assert (t[outside] == -1024.0).all(), f"{k}: rows outside the table were written"
    snap = {k: getattr(dw.ct, k).clone() for k in ("h", "q", "k", "v", "m", "l", "o")}
    blk = torch.from_numpy(np.concatenate([ids[3 + 56:3 + 72], ids[92 + 50:92 + 66]])[::-1].copy()).cuda()
    ws = dw.ctx.alloc_workspace(lacache.OP_BLOCK_STEP, table)
    dw.ctx.block_step(dw.weights, blk, table, dw.ct, ws)
    torch.cuda.synchronize()
    blockrows = np.r_[3 + 56:3 + 72, 92 + 50:92 + 66]
    keep = np.setdiff1d(np.arange(n_rows), blockrows)
    for k in ("h", "q", "k", "v"):
        a, b_ = getattr(dw.ct, k).float().cpu().numpy(), snap[k].float().cpu().numpy()
        assert np.array_equal(a[keep], b_[keep]), f"{k}: non-block rows changed"
    for k in ("m", "l", "o"):
        assert torch.equal(getattr(dw.ct, k), snap[k]), f"{k}: FACache was written by a block step"


def test_block_covering_the_whole_sequence():
    """No invariant rows (N = B): the step is plain attention over the block."""
    wl = synth.custom("u_empty", dtype="bf16", d_model=512, n_heads=4, head_dim=128, vocab=300,
                      prompt_lens=(0, 0), gen_len=32, block_size=32, block_idx=(0, 0), steps=1, seed=34)
    _run_full(wl, 1)


def test_out_of_range_token_id_reads_zero_row_and_sets_flag():
    wl = synth.custom("bad_id", dtype="f32", d_model=256, n_heads=4, head_dim=64, vocab=100,
                      prompt_lens=(20,), gen_len=16, block_size=16, block_idx=(0,), steps=1, embed_std=0.02, seed=35)
    dw = DeviceWorkload(wl)
    dw.prefill()
    assert dw.ctx.read_device_status() == 0
    blk = dw.next_block_ids()
    bad = blk.clone()
    bad[3] = wl.vocab + 5
    dw.block_step(bad)
    flags = dw.ctx.read_device_status()
    assert flags & lacache.DEVFLAG_BAD_TOKEN_ID
    assert dw.ctx.read_device_status() == 0          # reading clears the word
    off, n, bs, be = dw.table[0]
    assert torch.count_nonzero(dw.ct.h[off + bs + 3]) == 0
    assert torch.count_nonzero(dw.ct.q[off + bs + 3]) == 0
    assert torch.isfinite(dw.ct.out).all()


def test_invalid_arguments_are_rejected_before_any_launch():
    wl = synth.WORKLOADS["tiny"]
    dw = DeviceWorkload(wl)
    dw.prefill()
    torch.cuda.synchronize()
    before = dw.ct.out.clone()
    blk = dw.next_block_ids()
    bad_tables = [
        [(0, 128, 80, 80)],          # empty block
        [(0, 128, 90, 80)],          # block_end < block_start
        [(0, 128, 80, 129)],         # block past the sequence
        [(0, 129, 80, 96)],          # rows past n_rows / max_seq_len
        [(-1, 128, 80, 96)],         # negative offset
        [(0, 64, 0, 16), (32, 64, 32, 48)],   # overlapping samples
        [(0, 128, 0, 129)],
    ]
    for t in bad_tables:
        with pytest.raises(lacache.LaCacheError) as ei:
            dw.ctx.block_step(dw.weights, blk, t, dw.ct, dw.ws)
        assert ei.value.status in (lacache.ERR_INVALID_ARG, lacache.ERR_UNSUPPORTED), t
    with pytest.raises(lacache.LaCacheError) as ei:
        dw.ctx.block_step(dw.weights, blk, dw.table, dw.ct, None)
    assert ei.value.status == lacache.ERR_WORKSPACE
    with pytest.raises(lacache.LaCacheError) as ei:
        dw.ctx.block_step(dw.weights, blk, [(0, 160, 0, 160)], dw.ct, dw.ws)
    # Block-boundary refresh: proj and seqs must describe the same samples.
    for proj, seqs in (([(0, 100, 80, 96)], [(0, 128, 96, 112)]), ([(8, 120, 80, 96)], [(0, 128, 96, 112)])):
        with pytest.raises(lacache.LaCacheError) as ei:
            dw.ctx.refresh_block(dw.weights, blk, proj, seqs, dw.ct, workspace=dw.ws)
        assert ei.value.status == lacache.ERR_INVALID_ARG, (proj, seqs)
    torch.cuda.synchronize()
    assert torch.equal(before, dw.ct.out), "a rejected call wrote the output"
