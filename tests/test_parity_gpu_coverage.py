"""GPU parity of the kernel instantiations that only some shapes reach.

* Blocks of 96 and 128 keys (the block table accepts up to 128): the
  65-127-token projection, the 128-key instantiations of the small-launch
  attention (block-row partials and invariant rows in one launch), the
  invariant-row kernel beside the streaming block-row kernel, the
  block-boundary refresh and the DualCache attention.
* The head_dim-128 streaming block-row kernel (2- and 4-stage rings) and the
  streaming invariant-row kernel for blocks of 32 and 64 keys, every row.
* Cache rows past 2^31 / (H d_h), where the cache offsets need 64 bits.

Each case runs through the C ABI, is compared element by element with the
fp64 oracle and with the attention over the GPU's own cache values
(tests/attn_check.py), and asserts from the library's launch log
(LACACHE_LOG) that the kernel instantiations it is meant to reach ran.
"""

import re
import sys

import numpy as np
import pytest
import torch

import attn_check
import oracle
from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload
from helpers import cfg_of, check_cache_values, check_lse, check_output, host
from test_parity_gpu import _compare_refresh, _run_full

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _launched(capfd):
    """Kernel instantiations launched since the last read (from the launch
    log; the 16-bit cache type _Float16 reads as "half").  What the test
    printed meanwhile is passed through."""
    out, err = capfd.readouterr()
    with capfd.disabled():
        sys.stdout.write(out)
        sys.stdout.flush()
    names = re.findall(r"lacache launch: (.+?) grid \d+", err)
    return set(names)


def _expect(names, *patterns):
    for p in patterns:
        assert any(re.fullmatch(p, n) for n in names), f"no launch of {p}; launched: {sorted(names)}"


def _dualcache_every_row(dw, what):
    """DualCache attention over the current caches, every block row against the
    oracle and against the attention over the GPU's own q/k/v."""
    wl = dw.wl
    cfg = cfg_of(wl)
    crow = np.concatenate([off + np.arange(bs, be) for (off, n, bs, be) in dw.table])
    q_block = dw.ct.q.index_select(0, torch.from_numpy(crow).to("cuda")).contiguous()
    out_block = torch.empty(q_block.shape, dtype=dw.ctx.torch_dtype, device="cuda")
    lse_block = torch.empty(q_block.shape[:2], dtype=torch.float32, device="cuda")
    ws = dw.ctx.alloc_workspace(lacache.OP_DUALCACHE_ATTN, dw.table)
    dw.ctx.dualcache_attn(q_block, dw.ct.k, dw.ct.v, dw.table, out_block, lse_block, ws)
    torch.cuda.synchronize()
    ref = oracle.full_recompute(dw.params, cfg, dw.ids_host, dw.table)
    check_output(host(out_block), ref["out"][crow], wl.dtype, f"{what} out")
    check_lse(host(lse_block), ref["lse"][crow], wl.dtype, f"{what} lse")
    at = attn_check.check_block_query(q_block, dw.ct.k, dw.ct.v, dw.table, out_block, lse_block, cfg, what, wl.dtype)
    _say(f"[parity] {what} ok, attention-only {at}")


def _block_boundary(dw, seed, what):
    """lacache_refresh_block at the boundary to the next block: the finished
    block's rows get their final ids, the table moves one block on; every row,
    cache entry and FACache pair against the oracle's refresh of the new ids."""
    wl = dw.wl
    cfg = cfg_of(wl)
    rng = np.random.default_rng([20261202, seed])
    ids_new = np.array(dw.ids_host, copy=True)
    proj = dw.table
    for (off, n, bs, be) in proj:
        ids_new[off + bs:off + be] = rng.integers(0, wl.vocab, size=be - bs)
    proj_ids = np.concatenate([ids_new[off + bs:off + be] for (off, n, bs, be) in proj]).astype(np.int32)
    new_table = [(off, n, be, min(n, be + (be - bs))) for (off, n, bs, be) in proj]
    ws = dw.ctx.alloc_workspace(lacache.OP_REFRESH_BLOCK, proj)
    dw.ctx.refresh_block(dw.weights, torch.from_numpy(proj_ids).cuda(), proj, new_table, dw.ct, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.refresh(dw.params, cfg, ids_new, new_table)
    dw.table = new_table
    dw.ids_host = ids_new
    st = _compare_refresh(dw, ref, what)
    at = attn_check.check_all(dw.ct, dw.table, cfg, "refresh", what, wl.dtype)
    _say(f"[parity] {what} ok {st}, attention-only {at}")


# ---------------------------------------------------------------------------
# Blocks of 96 and 128 keys
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["one", "three"])
@pytest.mark.parametrize("block", [96, 128])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_blocks_every_row(dtype, head_dim, block, layout, monkeypatch, capfd):
    """Refresh, two steps, DualCache and the block-boundary refresh with blocks
    of 96 or 128 keys, every row.  "one": one sample (96 block tokens: the
    65-127-token projection; 128: the GEMM projection); "three": three ragged
    samples, one block at position 0."""
    monkeypatch.setenv("LACACHE_LOG", "1")
    d_model = (512 if head_dim == 128 else 256) if dtype == "f32" else 512
    if layout == "one":
        prompts, idx = (70,), (1,)
    else:
        prompts, idx = (37, 150, 5), (1, 0, 1)
    wl = synth.custom(f"blocks{block}_{dtype}_h{head_dim}_{layout}", dtype=dtype, d_model=d_model, n_heads=4,
                      n_kv_heads=2, head_dim=head_dim, vocab=1500, prompt_lens=prompts, gen_len=3 * block,
                      block_size=block, block_idx=idx, steps=2, embed_std=1.0 if dtype == "bf16" else 0.02,
                      seed=80 + block + head_dim)
    _say(f"[parity] {wl.name}: table {wl.table()}")
    dw = _run_full(wl, 2)
    names = _launched(capfd)
    T = "half, unsigned short" if dtype == "bf16" else "float, float"
    _expect(names, rf"lc::attn_ab_kernel<{T}, {head_dim}, 128>", rf"lc::merge_kernel<{T}, {head_dim}>")
    if dtype == "bf16" and layout == "one" and block == 96:
        _expect(names, r"lc::qkv_fused_kernel<.*>")
    if dtype == "bf16" and (layout == "three" or block == 128):
        _expect(names, r"lc::qkv_prep_kernel<\d+>", r"lc::qkv_gemm_packed(_wide)?_kernel<.*>")
    _dualcache_every_row(dw, f"{wl.name} dualcache")
    _block_boundary(dw, 90 + block, f"{wl.name} block refresh")
    names = _launched(capfd)
    _say(f"[parity] {wl.name} launched {sorted(names)}")
    _expect(names, rf"lc::block_rows_kernel<{T}, {head_dim}>")
    if dtype == "bf16":
        _expect(names, rf"lc::refresh_stream_kernel<unsigned short, {head_dim}, [12], 2>")
    else:
        _expect(names, rf"lc::refresh_attn_kernel<float, float, {head_dim}>")
    assert dw.ctx.read_device_status() == 0


@pytest.mark.parametrize("head_dim", [64, 128])
def test_large_blocks_streaming_launch(head_dim, monkeypatch, capfd):
    """Blocks of 128 keys in a launch large enough for whole-sequence block-row
    chunks (8 samples x 8 heads x 4 row groups = 256 workgroups): the streaming
    block-row kernel writes O and LSE itself and the 128-key invariant-row
    kernel runs beside it (no merge).  Every row; DualCache on the same table."""
    monkeypatch.setenv("LACACHE_LOG", "1")
    rng = np.random.default_rng([20261202, 75, head_dim])
    prompts = tuple(int(x) for x in rng.integers(100, 400, size=8))
    wl = synth.custom(f"blocks128_stream_h{head_dim}", dtype="bf16", d_model=1024 if head_dim == 128 else 512,
                      n_heads=8, n_kv_heads=8, head_dim=head_dim, vocab=2000, prompt_lens=prompts, gen_len=384,
                      block_size=128, steps=2, seed=76 + head_dim)
    _say(f"[parity] {wl.name}: table {wl.table()}")
    dw = _run_full(wl, 2)
    _dualcache_every_row(dw, f"{wl.name} dualcache")
    names = _launched(capfd)
    _say(f"[parity] {wl.name} launched {sorted(names)}")
    _expect(names, rf"lc::block_rows_stream_kernel<unsigned short, {head_dim}, 4>",
            rf"lc::invariant_rows_kernel<half, unsigned short, {head_dim}, 128>")


# ---------------------------------------------------------------------------
# head_dim 128 streaming kernels, every row
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["b32_equal", "b64_ragged"])
def test_streaming_kernels_head128_every_row(case, monkeypatch, capfd):
    """b32_equal: 32 samples of 632 tokens, blocks of 32, 8 heads of 128:
    256 whole-sequence block-row workgroups (4-stage ring) and more than 2048
    (64-row tile, head) invariant items in equal segments (the 32-key
    streaming invariant-row kernel, four waves per workgroup).  b64_ragged:
    28 samples of 628..828 tokens, blocks of 64: 448 block-row workgroups
    (2-stage ring, two per CU) and 192-row segments of the 64-key streaming
    invariant-row kernel."""
    monkeypatch.setenv("LACACHE_LOG", "1")
    if case == "b32_equal":
        prompts, block, gen = (568,) * 32, 32, 64
    else:
        rng = np.random.default_rng([20261202, 74])
        prompts, block, gen = tuple(int(x) for x in rng.integers(500, 701, size=28)), 64, 128
    wl = synth.custom(f"stream_h128_{case}", dtype="bf16", d_model=1024, n_heads=8, head_dim=128, vocab=3000,
                      prompt_lens=prompts, gen_len=gen, block_size=block, steps=1, seed=73)
    dw = _run_full(wl, 1)
    names = _launched(capfd)
    _say(f"[parity] {wl.name} launched {sorted(names)}")
    nst, nks = (4, 1) if case == "b32_equal" else (2, 2)
    _expect(names, rf"lc::block_rows_stream_kernel<unsigned short, 128, {nst}>",
            rf"lc::invariant_stream_kernel<unsigned short, 128, {nks}, 4>")


# ---------------------------------------------------------------------------
# Cache rows whose element offsets exceed 2^31
# ---------------------------------------------------------------------------

def test_cache_rows_past_32bit_element_offsets(monkeypatch, capfd):
    """A sample whose rows start past row 2^31 / (H d_h) = 4,194,304 (H d_h =
    512): its q offsets exceed 2^31 elements.  Refresh (GEMM projection) and a
    block step of 32 tokens (the fused projection for at most 64 tokens, whose
    q/k/v offsets are 64-bit), every row of both samples against the oracle.
    The caches hold 4.2 M rows (about 20 GB)."""
    monkeypatch.setenv("LACACHE_LOG", "1")
    wl = synth.custom("offset64", dtype="bf16", d_model=512, n_heads=4, n_kv_heads=1, head_dim=128, vocab=1000,
                      prompt_lens=(60, 140), gen_len=64, block_size=16, block_idx=(1, 2), steps=1, seed=91)
    H, d = wl.n_heads, wl.head_dim
    R = (1 << 31) // (H * d) + 1000
    compact = wl.table()
    (o0, n0, bs0, be0), (o1, n1, bs1, be1) = compact
    table = [(0, n0, bs0, be0), (R, n1, bs1, be1)]
    n_rows = R + n1
    assert (R + bs1) * H * d > 2 ** 31
    _say(f"[parity] offset64: table {table}, n_rows {n_rows}")
    dw = DeviceWorkload(wl, n_rows=n_rows)
    cfg = cfg_of(wl)
    ids_c = synth.initial_ids(wl)
    ids = np.zeros(n_rows, np.int32)
    ids[0:n0] = ids_c[o0:o0 + n0]
    ids[R:R + n1] = ids_c[o1:o1 + n1]
    dw.ctx.prefill_cache(dw.weights, torch.from_numpy(ids).cuda(), table, dw.ct,
                         workspace=dw.ctx.alloc_workspace(lacache.OP_PREFILL, table))
    rng = np.random.default_rng([20261202, 92])
    for (_, _, bs, be), off in zip(table, (0, R)):
        ids[off + bs:off + be] = rng.integers(0, wl.vocab, size=be - bs)
    blk = np.concatenate([ids[off + bs:off + be] for (off, _, bs, be) in table]).astype(np.int32)
    dw.ctx.block_step(dw.weights, torch.from_numpy(blk).cuda(), table, dw.ct,
                      dw.ctx.alloc_workspace(lacache.OP_BLOCK_STEP, table))
    torch.cuda.synchronize()
    ids_c2 = np.concatenate([ids[0:n0], ids[R:R + n1]])
    ref = oracle.full_recompute(dw.params, cfg, ids_c2, compact)
    for (off, n, bs, be), (oc, _, _, _) in zip(table, compact):
        sl = slice(off, off + n)
        rows = slice(oc, oc + n)
        assert np.array_equal(host(dw.ct.h[sl]), ref["h"][rows]), f"EmbedCache rows at {off}"
        for key in ("q", "k", "v"):
            check_cache_values(host(getattr(dw.ct, key)[sl]), ref[key][rows], "bf16", f"{key} at {off}")
        st = check_output(host(dw.ct.out[sl]), ref["out"][rows], "bf16", f"out at {off}")
        check_lse(host(dw.ct.lse[sl]), ref["lse"][rows], "bf16", f"lse at {off}")
        _say(f"[parity] offset64 sample at row {off}: {st}")
    names = _launched(capfd)
    _say(f"[parity] offset64 launched {sorted(names)}")
    _expect(names, r"lc::qkv_skinny_fused_kernel<128, \d+, \d+>")
    assert dw.ctx.read_device_status() == 0
