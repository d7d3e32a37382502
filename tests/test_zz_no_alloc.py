"""lacache_block_step_noalloc against lacache_block_step.

The no-allocation entry point runs the same kernels on the library's static
scratch instead of a caller workspace.  Two calls in a row through the C ABI,
the second on a smaller input (so the scratch holds the first call's
contents), must give the same caches, output and LSE as lacache_block_step
on the same inputs (bitwise: same kernels, same work split), and match the
fp64 oracle at the output bar.  A table whose scratch need exceeds the static
size is rejected before any launch.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload
from helpers import cfg_of, check_lse, check_output, host

pytestmark = pytest.mark.gpu

STATIC_SCRATCH_BYTES = 32 << 20


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _clone(ctx, ct):
    c = ctx.alloc_cache(ct.n_rows)
    for k in ("h", "q", "k", "v", "m", "l", "o", "out", "lse"):
        getattr(c, k).copy_(getattr(ct, k))
    return c


def _one_call(wl, what):
    """Prefill, then one step twice: lacache_block_step on one copy of the
    caches, lacache_block_step_noalloc on another."""
    _say(f"[noalloc] {what}: {wl.name} table {wl.table()[:3]}... M {wl.block_tokens}")
    dw = DeviceWorkload(wl)
    need = dw.ctx.workspace_size(lacache.OP_BLOCK_STEP, dw.table)
    dw.prefill()
    torch.cuda.synchronize()
    ct2 = _clone(dw.ctx, dw.ct)
    blk = dw.next_block_ids()
    dw.block_step(blk)
    dw.ctx.block_step_noalloc(dw.weights, blk, dw.table, ct2)
    torch.cuda.synchronize()
    for k in ("h", "q", "k", "v", "out", "lse", "m", "l", "o"):
        # bitwise: the FACache entries of block rows are never written and may
        # hold any bits, NaN patterns included (which torch.equal calls unequal)
        a, b = getattr(dw.ct, k), getattr(ct2, k)
        bits = torch.int16 if a.element_size() == 2 else torch.int32
        assert torch.equal(a.view(bits), b.view(bits)), f"{what}: {k} differs from lacache_block_step"
    ref = oracle.full_recompute(dw.params, cfg_of(wl), dw.ids_host, dw.table)
    rows = np.concatenate([np.arange(off, off + n) for (off, n, _, _) in dw.table])
    st = check_output(host(ct2.out)[rows], ref["out"][rows], wl.dtype, f"{what} out")
    check_lse(host(ct2.lse)[rows], ref["lse"][rows], wl.dtype, f"{what} lse")
    _say(f"[noalloc] {what}: bitwise equal to lacache_block_step, oracle {st}, workspace bound {need} bytes")
    return need


def test_noalloc_step_matches_block_step_on_two_calls():
    # First call: 6 samples, 192 block tokens (the prep + GEMM projection and
    # the split-KV partials both use the scratch).
    big = synth.custom("noalloc_big", dtype="bf16", d_model=1024, n_heads=8, n_kv_heads=4, head_dim=128, vocab=2000,
                       prompt_lens=(300, 41, 512, 7, 260, 100), gen_len=64, block_size=32, steps=1, seed=201)
    need_big = _one_call(big, "call 1")
    # Second call, smaller: one sample, 16 block tokens (the fused projection
    # for at most 64 tokens; partials only).
    small = synth.custom("noalloc_small", dtype="bf16", d_model=512, n_heads=4, head_dim=64, vocab=900,
                         prompt_lens=(90,), gen_len=32, block_size=16, block_idx=(1,), steps=1, seed=202)
    need_small = _one_call(small, "call 2")
    assert need_small < need_big <= STATIC_SCRATCH_BYTES


def test_noalloc_rejects_tables_beyond_the_static_scratch():
    # 64 samples x 128 block tokens at d_model 2048: the projection's
    # activation tiles alone need 32 MiB, beyond the static scratch.
    wl = synth.custom("noalloc_too_big", dtype="bf16", d_model=2048, n_heads=16, head_dim=128, vocab=500,
                      prompt_lens=(0,) * 64, gen_len=128, block_size=128, block_idx=(0,) * 64, steps=1, seed=203)
    ctx = lacache.context_for(wl)
    need = ctx.workspace_size(lacache.OP_BLOCK_STEP, wl.table())
    assert need > STATIC_SCRATCH_BYTES
    dw = DeviceWorkload(wl, ctx=ctx)
    dw.ct.out.fill_(7.0)
    torch.cuda.synchronize()
    blk = torch.zeros(wl.block_tokens, dtype=torch.int32, device="cuda")
    with pytest.raises(lacache.LaCacheError) as ei:
        ctx.block_step_noalloc(dw.weights, blk, dw.table, dw.ct)
    assert ei.value.status == lacache.ERR_UNSUPPORTED
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((dw.ct.out == 7.0).all()), "a rejected call wrote the output"
