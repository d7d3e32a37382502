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

import oracle
from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload
from helpers import cfg_of, check_cache_values, check_lse, check_output, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _facache_pair(dw, rows):
    m, l, o = host(dw.ct.m)[rows], host(dw.ct.l)[rows], host(dw.ct.o_acc)[rows]
    return o / l[..., None], m + np.log(l)


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


def _run_full(wl, steps):
    _say(f"[parity] {wl.name}: dtype {wl.dtype} D {wl.d_model} H {wl.n_heads}x{wl.head_dim} "
         f"batch {wl.batch} seq_lens {wl.seq_lens[:4]}... block {wl.block_size} seed {wl.seed}")
    dw = DeviceWorkload(wl)
    cfg = cfg_of(wl)
    dw.prefill()
    torch.cuda.synchronize()
    ref = oracle.refresh(dw.params, cfg, dw.ids_host, dw.table)
    st = _compare_refresh(dw, ref, f"{wl.name} refresh")
    _say(f"[parity] {wl.name} refresh ok {st}")
    for s in range(1, steps + 1):
        blk = dw.next_block_ids()
        dw.block_step(blk)
        torch.cuda.synchronize()
        ref = oracle.full_recompute(dw.params, cfg, dw.ids_host, dw.table)
        st = _compare_step(dw, ref, f"{wl.name} step {s}")
        _say(f"[parity] {wl.name} step {s} ok {st}")
    return dw


def test_tiny_fp32_refresh_and_steps():
    _run_full(synth.WORKLOADS["tiny"], 3)


def test_small_bf16_ragged_batch():
    # Three samples: ragged lengths (not multiples of any tile), a block at the
    # very start, a block at the very end, and grouped KV heads.
    wl = synth.custom("small_bf16_ragged", dtype="bf16", d_model=512, n_heads=4, n_kv_heads=2, head_dim=128,
                      vocab=3000, prompt_lens=(37, 150, 5), gen_len=70, block_size=14, block_idx=(2, 0, 4),
                      steps=3, seed=21)
    _run_full(wl, 3)


def test_small_fp32_head64_multi_tile():
    wl = synth.custom("small_fp32_h64", dtype="f32", d_model=256, n_heads=4, head_dim=64, vocab=700,
                      prompt_lens=(300, 77), gen_len=96, block_size=32, block_idx=(1, 2), steps=2,
                      embed_std=0.02, seed=22)
    _run_full(wl, 2)


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
