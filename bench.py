#!/usr/bin/env python3
"""Benchmark of the exact layer-0 cached block step on one MI355X.

One "step" = one lacache_block_step over the whole batch: block-token
embedding (EmbedCache), fused RMSNorm + QKV + RoPE + cache write, block-row
attention over [prefix | block | suffix] keys, invariant rows merged from the
FACache state, and the final O / LSE of every row.

Workload: the LLaDA-8B-shaped first layer (d_model 4096, 32 heads of 128,
vocabulary 126464, bf16 with fp32 accumulation), batch 1, prompt 512 + gen
256 tokens, blocks of 32, current block 3; the inner steps cycle through 20
seeded edits of 2..8 block tokens.  Inputs are synthetic (seeded Gaussian
parameters, uniform ids) and resident in HBM before timing starts.

Cold-cache protocol: `--sets` independent copies of the layer (weights,
caches, workspace) are used round-robin, so every step streams its 100 MB of
W_qkv from HBM rather than from the 256 MB Infinity Cache.  A warm figure
(one set) is reported beside it.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
MFMA_FP32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llada8b")
    p.add_argument("--sets", type=int, default=4, help="rotating buffer sets (cold-cache protocol); must divide 20")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--refresh-reps", type=int, default=8, help="timed refresh calls (0: skip the refresh timing)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 512 MiB device copy (3 times): the reference for FETCH_SIZE/WRITE_SIZE")
    p.add_argument("--ffn-rows", default="768,8192",
                   help="rows of the per-group FP8 FFN measurement (LLaDA-8B FFN shape); empty: skip it")
    p.add_argument("--ffn-only", action="store_true", help="only the FP8 FFN measurement (its JSON object)")
    p.add_argument("--no-layer", action="store_true", help="skip the layer-finish and sampler measurement")
    p.add_argument("--layer-only", action="store_true", help="only the layer-finish and sampler measurement")
    p.add_argument("--no-multilayer", action="store_true", help="skip the approximate deeper-layer reuse measurement")
    p.add_argument("--multilayer-only", action="store_true", help="only the approximate deeper-layer reuse measurement")
    p.add_argument("--no-flashdllm", action="store_true", help="skip the selective update / verify measurement")
    return p.parse_args()


KERNEL_SOURCES = {
    "qkv": ["exact_attention_state_amd/csrc/qkv.hip"],
    "qkv_prep": ["exact_attention_state_amd/csrc/gemm.hip"],
    "qkv_gemm": ["exact_attention_state_amd/csrc/gemm.hip"],
    "block_rows": ["exact_attention_state_amd/csrc/attn.hip"],
    "invariant_rows": ["exact_attention_state_amd/csrc/attn.hip"],
    "attn": ["exact_attention_state_amd/csrc/attn.hip"],
}
COMMON_SOURCES = ["exact_attention_state_amd/csrc/common.h", "exact_attention_state_amd/csrc/internal.h"]
def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}_step.json")


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []) + COMMON_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter runs, if the kernel is unchanged since."""
    try:
        with open(traffic_file(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or rec.get("workload") != workload or k.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 512 * 1024 * 1024
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def stream_copy_gbs(dev, reps=5):
    """STREAM-style device copy of 512 MiB (read + write bytes per second, GB/s): the
    achievable bandwidth that the HBM-bound kernels are also compared with."""
    import torch
    n = 512 * 1024 * 1024
    src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def attention_summary(acc, kern):
    """The step's attention (block rows and invariant rows, with the merge of the
    block rows' partials where it runs) as one unit: algorithmic bytes over the
    summed average durations of its launches, against the HBM peak."""
    names = [k for k in ("attn", "block_rows", "invariant_rows", "merge") if k in kern]
    us = sum(kern[k]["us_avg"] for k in names)
    nbytes = acc["kernels"]["attn"]["bytes"]
    return {"kernels": names, "us": us, "algorithmic_bytes": nbytes,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS if us else None}


def projection_summary(acc, kern, peak_flops):
    """The step's projection (prep and GEMM, or the single fused launch): flops
    over the summed average durations, against the bf16 MFMA peak and against
    the attainable roofline min(peak, AI x HBM peak)."""
    names = [k for k in ("qkv", "qkv_prep", "qkv_gemm") if k in kern]
    us = sum(kern[k]["us_avg"] for k in names)
    flops = sum(acc["kernels"][k]["flops"] for k in names)
    nbytes = sum(acc["kernels"][k]["bytes"] for k in names)
    if not us:
        return None
    rate = flops / (us * 1e-6)
    attainable = min(peak_flops, flops / nbytes * HBM_PEAK_GBS * 1e9)
    return {"kernels": names, "us": us, "flops": flops, "algorithmic_bytes": nbytes,
            "mfma_frac": rate / peak_flops, "attainable_frac": rate / attainable}


def step_accounting(wl):
    """Work and algorithmic HBM bytes of one block step of workload `wl`, per kernel.

    Algorithmic bytes are what the step must move at least: W_qkv, gamma, the
    block rows' embedding rows and Q/K/V/h writes (qkv); Q of the block rows,
    K and V of every key, O and LSE of the block rows (block_rows, whose merge
    runs in the next kernel); Q and the FACache state (m, l, O~/l) of the
    invariant rows, their O and LSE (invariant_rows).  The split-KV partials
    are not counted: they are an artefact of the kernel split.
    """
    s = 2 if wl.dtype == "bf16" else 4          # parameter / output bytes
    c = 2 if wl.dtype == "bf16" else 4          # cache (ctype) bytes
    D, H, Hk, d, F = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.n_features
    M = sum(be - bs for (_, _, bs, be) in wl.table())
    pairs_c = pairs_e = pairs_a = pairs_b = 0
    a_bytes = b_bytes = 0
    for (_, n, bs, be) in wl.table():
        B = be - bs
        U = n - B
        pairs_a += H * B * n
        pairs_b += H * U * B
        pairs_e += H * n * n
        a_bytes += B * H * d * c + 2 * n * Hk * d * c + B * H * d * s + B * H * 4
        b_bytes += U * H * d * c + U * H * (2 * 4 + d * c) + U * H * d * s + U * H * 4
    pairs_c = pairs_a + pairs_b
    qkv_bytes = F * D * s + 2 * M * D * s + D * s + M * F * c + M * 4
    kern = {"block_rows": dict(bytes=a_bytes, flops=4 * d * pairs_a),
            "invariant_rows": dict(bytes=b_bytes, flops=4 * d * pairs_b),
            # small steps run both in one launch
            "attn": dict(bytes=a_bytes + b_bytes, flops=4 * d * (pairs_a + pairs_b))}
    skinny = 1 <= M <= 64 and D // 512 in (1, 2, 4, 8, 16) and wl.vocab * D * 2 < 2 ** 32
    if wl.dtype == "bf16" and D % 512 == 0 and skinny:
        # At most 64 tokens: one launch streams the packed fp16 weight,
        # gathers the embedding rows, writes the EmbedCache rows and Q/K/V
        # (bound by the weight's HBM stream).
        kern["qkv_gemm"] = dict(bytes=F * D * 2 + 2 * M * D * s + D * s + M * F * c, flops=2 * M * F * D)
    elif wl.dtype == "bf16" and D % 512 == 0 and M >= 128:
        # Prep (embedding rows in, EmbedCache rows and the fp16 activations
        # out), then the GEMM over the packed fp16 weight (activations in,
        # Q/K/V out; the matrix cores bound it).
        kern["qkv_prep"] = dict(bytes=2 * M * D * s + D * s + M * D * 2 + M * 4, flops=0)
        kern["qkv_gemm"] = dict(bytes=F * D * 2 + M * D * 2 + M * F * c, flops=2 * M * F * D)
    else:
        kern["qkv"] = dict(bytes=qkv_bytes, flops=2 * M * F * D)
    return dict(M=M, pairs_computed=pairs_c, pairs_equiv=pairs_e, kernels=kern,
                qkv_bytes=qkv_bytes, attn_bytes=a_bytes + b_bytes)


def refresh_accounting(wl):
    """Work of one refresh (lacache_prefill_cache): the projection of every
    row and full bidirectional attention per sample (4 d flops per
    query-key pair), plus the FACache written for the invariant rows."""
    D, H, Hk, d, F = wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.n_features
    T = sum(n for (_, n, _, _) in wl.table())
    pairs = sum(H * n * n for (_, n, _, _) in wl.table())
    return {"rows": T, "attn_flops": 4 * d * pairs, "proj_flops": 2 * T * F * D, "pairs": pairs}


def measure_refresh(ctx, sets, base, stream, dev, reps, acc, wl, blk):
    """Time the refresh on the rotating sets: lacache_prefill_cache (every
    row re-projected) as whole calls with events on the launch stream, then
    the same calls with every kernel bracketed by events (per-kernel
    averages); and lacache_refresh_block (the block boundary: only the
    finished block's rows re-projected, here the current block's rows with
    the step ids `blk`, then the full refresh attention)."""
    import torch
    from exact_attention_state_amd import lacache
    ids_dev = base.upload_ids(base.ids_host)
    ws = ctx.alloc_workspace(lacache.OP_PREFILL, base.table, dev)

    def call(r):
        s = sets[r % len(sets)]
        ctx.prefill_cache(s.weights, ids_dev, base.table, s.ct, workspace=ws, stream=stream)

    call(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record(stream)
        call(r + 1)
        evs[r][1].record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    ctx.profile(True)
    ctx.profile_read()
    for r in range(reps):
        call(r + 1)
    torch.cuda.synchronize()
    prof = ctx.profile_read()
    ctx.profile(False)
    kern = {k: v[0] * 1e3 / v[1] for k, v in prof.items() if v[1]}
    ws_b = ctx.alloc_workspace(lacache.OP_REFRESH_BLOCK, base.table, dev)

    def call_b(r):
        s = sets[r % len(sets)]
        ctx.refresh_block(s.weights, blk, base.table, base.table, s.ct, workspace=ws_b, stream=stream)

    call_b(0)
    torch.cuda.synchronize()
    evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for r in range(reps):
        evb[r][0].record(stream)
        call_b(r + 1)
        evb[r][1].record(stream)
    torch.cuda.synchronize()
    usb = sorted(a.elapsed_time(b) * 1e3 for a, b in evb)
    ra = refresh_accounting(wl)
    peak = (MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS) * 1e12
    t_attn = kern.get("refresh_attn")
    out = {"us_per_refresh": us[len(us) // 2], "us_per_refresh_min": us[0], "calls": reps,
           "us_per_block_refresh": usb[len(usb) // 2],
           "kernels_us_avg_per_call": {k: v * prof[k][1] / reps for k, v in kern.items()},
           "attn_flops": ra["attn_flops"],
           "attn_mfma_frac": None if not t_attn else ra["attn_flops"] / (t_attn * prof["refresh_attn"][1] / reps * 1e-6) / peak}
    log(f"[bench] refresh: {out['us_per_refresh']:.1f} us per call (block-boundary refresh "
        f"{out['us_per_block_refresh']:.1f} us); kernels per call "
        + ", ".join(f"{k} {v:.1f} us" for k, v in out["kernels_us_avg_per_call"].items())
        + (f"; attention at {out['attn_mfma_frac']:.3f} of MFMA peak" if out["attn_mfma_frac"] else ""))
    return out


def ffn_accounting(T, D, F):
    """Work and algorithmic HBM bytes of one FP8 FFN call per kernel: the
    AddNorm reads h and the attention output and writes r, the x codes and
    scales; the gate-up GEMM reads its FP8 weight once plus the x codes and
    writes the y codes and scales; the down GEMM reads its weight, the y
    codes, r, and writes out."""
    Mp = -(-T // 256) * 256
    return {"ffn_norm": dict(bytes=3 * T * D * 2 + D * 2 + Mp * D + Mp * D // 128 * 4, flops=0),
            "ffn_gate_up": dict(bytes=2 * F * D + Mp * D + Mp * D // 128 * 4 + Mp * F + Mp * F // 128 * 4,
                                flops=2 * T * D * 2 * F),
            "ffn_down": dict(bytes=D * F + Mp * F + Mp * F // 128 * 4 + 2 * T * D * 2, flops=2 * T * F * D)}


def measure_ffn(dev, rows_list, reps=20, n_sets=3):
    """The per-group FP8 FFN of a layer after the first at LLaDA-8B's shape
    (d_model 4096, d_ff 12288), for each row count: median time per call over
    `reps` calls cycling `n_sets` independent packed weight sets (150 MB each,
    so the set a call reads is not left in the 256 MB memory-side cache by the
    previous call), per-kernel averages from event-bracketed calls, and each
    GEMM's fraction of the dense FP8 matrix-core peak."""
    import numpy as np
    import torch
    from exact_attention_state_amd import lacache, synth
    D, F = 4096, synth.LLADA_D_FF
    ctx = lacache.Context(D, 32, 32, 128, 1000, 64, 5e5, 1e-5, 0.0, "bf16")
    p = synth.ffn_params(D, F, 2)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(dev)
    g = bf(p["gamma"])
    sets = []
    for i in range(n_sets):
        wg, wu, wd = bf(p["w_gate"]), bf(p["w_up"]), bf(p["w_down"])
        sets.append(ctx.ffn_pack_weights(F, wg, wu, wd))
        del wg, wu, wd
    stream = torch.cuda.Stream(device=dev)
    res = {"shape": {"d_model": D, "d_ff": F}, "protocol": f"cold ({n_sets} rotating packed weight sets)", "rows": {}}
    for T in rows_list:
        h, a = synth.ffn_inputs(T, D, 7)
        hd, ad = bf(h), bf(a)
        out, r = torch.empty_like(hd), torch.empty_like(hd)
        ws = ctx.ffn_workspace(F, T, True, dev)

        def call(i):
            ctx.ffn_fp8(F, g, sets[i % n_sets], hd, ad, out, r_out=r, workspace=ws, stream=stream)

        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            call(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = sorted(x.elapsed_time(y) * 1e3 for x, y in ev)[reps // 2]
        ctx.profile(True)
        ctx.profile_read()
        for i in range(reps):
            call(i)
        torch.cuda.synchronize()
        prof = ctx.profile_read()
        ctx.profile(False)
        acc = ffn_accounting(T, D, F)
        kern = {}
        for k in ("ffn_norm", "ffn_gate_up", "ffn_down"):
            ms, n = prof[k]
            t = ms * 1e3 / n
            e = {"us_avg": t, "hbm_frac": acc[k]["bytes"] / (t * 1e-6) / 1e9 / HBM_PEAK_GBS}
            if acc[k]["flops"]:
                e["fp8_mfma_frac"] = acc[k]["flops"] / (t * 1e-6) / (MFMA_FP8_PEAK_TFLOPS * 1e12)
                e["tflops"] = acc[k]["flops"] / (t * 1e-6) / 1e12
            kern[k] = e
        flops = sum(v["flops"] for v in acc.values())
        res["rows"][str(T)] = {"us_per_call": us, "tflops": flops / (us * 1e-6) / 1e12,
                               "fp8_mfma_frac": flops / (us * 1e-6) / (MFMA_FP8_PEAK_TFLOPS * 1e12),
                               "kernels": kern, "algorithmic_bytes": {k: v["bytes"] for k, v in acc.items()},
                               "flops": {k: v["flops"] for k, v in acc.items()}}
        log(f"[bench] FP8 FFN rows {T}: {us:.1f} us per call ({flops / (us * 1e-6) / 1e12:.0f} TFLOP/s); "
            + ", ".join(f"{k} {v['us_avg']:.1f} us" + (f" ({v['fp8_mfma_frac']:.3f} of FP8 peak)" if 'fp8_mfma_frac' in v else "")
                        for k, v in kern.items()))
        del hd, ad, out, r, ws
    assert ctx.read_device_status() == 0
    return res


def host_info():
    """The host the oracle baseline runs on: CPU model, cores, NumPy and its BLAS."""
    import numpy as np
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"library": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads")}
                for i in threadpool_info()]
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": affinity,
            "numpy": np.__version__, "blas": blas}


def cpu_baseline(wl, budget_s, t_step_s):
    """Time the fp64 oracle on the host cores, on the same workload.

    The baseline is the oracle's definition of the step's result: a full
    layer-0 recompute of every row (oracle.full_recompute: embedding, RMSNorm,
    QKV, RoPE, bidirectional attention), which gives what one cached block
    step outputs.  `value` is the step's query-key pairs (the GPU metric's
    unit) per second of that recompute; the pairs the recompute itself
    evaluates (H N^2 per sample) per second and the ratio to the GPU step are
    beside it.  The oracle's plain fp64 cached step (oracle.cached_step, the
    method written out) is timed too."""
    import numpy as np
    import oracle
    from exact_attention_state_amd import synth
    info = host_info()
    threads = max([b["threads"] or 1 for b in info["blas"]] or [1])
    p = synth.params(wl)
    cfg = oracle.Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)
    ids = synth.initial_ids(wl)
    acc = step_accounting(wl)
    # The definition, on the ids of the first inner step.
    ids1, blk = synth.step_ids(wl, ids, 1)
    n_full, t_full = 0, 0.0
    while n_full < 3 and (n_full == 0 or t_full < budget_s / 2):
        t0 = time.perf_counter()
        oracle.full_recompute(p, cfg, ids1, wl.table())
        t_full += time.perf_counter() - t0
        n_full += 1
    sec_full = t_full / n_full
    # The method written out in fp64: refresh, then cached steps.
    t0 = time.perf_counter()
    cache = oracle.refresh(p, cfg, ids, wl.table())
    t_refresh = time.perf_counter() - t0
    steps, t_steps = 0, 0.0
    while t_steps < budget_s / 2 and steps < wl.steps:
        ids, blk = synth.step_ids(wl, ids, steps + 1)
        t0 = time.perf_counter()
        res = oracle.cached_step(p, cfg, cache, blk, wl.table())
        t_steps += time.perf_counter() - t0
        cache.update({k: res[k] for k in ("h", "q", "k", "v")})
        steps += 1
    sec_cached = t_steps / max(steps, 1)
    return {"value": acc["pairs_computed"] / sec_full, "unit": "query-key pairs/s",
            "cores": int(min(threads, info["affinity_cores"] or threads)), "kind": "oracle",
            "sample": f"{n_full} full layer-0 recomputes (oracle.full_recompute, fp64 NumPy) of the {wl.name} workload "
                      f"after its first inner step, {sec_full:.3f} s each; value = the step's {acc['pairs_computed']} "
                      f"query-key pairs per recompute second",
            "s_per_step_full_recompute": sec_full,
            "pairs_equiv_per_s": acc["pairs_equiv"] / sec_full,
            "ratio_to_gpu_step": sec_full / t_step_s,
            "cached_step": {"ms_per_step": sec_cached * 1e3, "steps": steps, "refresh_s": t_refresh,
                            "pairs_per_s": acc["pairs_computed"] / sec_cached},
            "host": info}


def layer_accounting(T, D, HD, F):
    """Work and algorithmic HBM bytes of one layer finish call per kernel (bf16)."""
    return {"layer_oproj": dict(flops=2 * T * HD * D, bytes=2 * (D * HD + T * HD + 2 * T * D)),
            "layer_norm": dict(flops=0, bytes=2 * (2 * T * D + D)),
            "layer_gate_up": dict(flops=2 * T * D * 2 * F, bytes=2 * (2 * F * D + T * D + T * F)),
            "layer_down": dict(flops=2 * T * F * D, bytes=2 * (D * F + T * F + 2 * T * D))}


def sampler_accounting(M, D, V):
    return {"sampler_norm": dict(flops=0, bytes=2 * (2 * M * D + D)),
            "sampler_lmhead": dict(flops=2 * M * V * D, bytes=2 * (V * D + M * D) + 4 * M * V),
            "sampler_softmax": dict(flops=0, bytes=4 * M * V + 8 * M)}


def _kernel_fracs(acc, prof):
    out = {}
    for k, a in acc.items():
        ms, n = prof[k]
        t = ms * 1e3 / max(n, 1)
        e = {"us_avg": t, "hbm_frac": a["bytes"] / (t * 1e-6) / 1e9 / HBM_PEAK_GBS}
        if a["flops"]:
            e["bf16_mfma_frac"] = a["flops"] / (t * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        out[k] = e
    return out


def measure_layer(dev, reps=20, n_sets=2):
    """The rest of layer 0 (lacache_layer_finish) over llada8b's 768 rows at
    LLaDA-8B's shape (d_model 4096, 32 x 128 heads, d_ff 12288), cycling
    `n_sets` weight sets (335 MB each, beyond the 256 MB memory-side cache),
    and the sampler (vocabulary 126464, a 1 GB lm-head) on the block's 32 rows
    (the cut) and on all 768 rows (no cut): median time per call and
    per-kernel averages from event-bracketed calls."""
    import numpy as np
    import torch
    from exact_attention_state_amd import lacache, synth
    wl = synth.WORKLOADS["llada8b"]
    T, D, F, V = wl.total_tokens, wl.d_model, synth.LLADA_D_FF, synth.LLADA_VOCAB
    HD = wl.n_heads * wl.head_dim
    ctx = lacache.context_for(wl)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(dev)
    stream = torch.cuda.Stream(device=dev)

    def timed_calls(call):
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            call(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = sorted(x.elapsed_time(y) * 1e3 for x, y in ev)[reps // 2]
        ctx.profile(True)
        ctx.profile_read()
        for i in range(reps):
            call(i)
        torch.cuda.synchronize()
        prof = ctx.profile_read()
        ctx.profile(False)
        return us, prof

    sets = []
    for i in range(n_sets):
        p = synth.layer_params(D, HD, F, i)
        sets.append([bf(p[k]) for k in ("w_o", "gamma", "w_gate", "w_up", "w_down")])
    h, _ = synth.ffn_inputs(T, D, 11)
    o = synth.ffn_inputs(T, HD, 12)[1]
    hd, od = bf(h), bf(o)
    out = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    r = torch.empty_like(out)
    ws = ctx.layer_workspace(F, T, True, dev)
    us, prof = timed_calls(lambda i: ctx.layer_finish(F, sets[i % n_sets], hd, od, out, r_out=r, workspace=ws,
                                                      stream=stream))
    acc = layer_accounting(T, D, HD, F)
    flops = sum(a["flops"] for a in acc.values())
    layer = {"shape": {"rows": T, "d_model": D, "heads_x_head_dim": HD, "d_ff": F},
             "protocol": f"cold ({n_sets} rotating weight sets)", "us_per_call": us,
             "bf16_mfma_frac": flops / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12),
             "kernels": _kernel_fracs(acc, prof), "flops": {k: a["flops"] for k, a in acc.items()},
             "algorithmic_bytes": {k: a["bytes"] for k, a in acc.items()}}
    log(f"[bench] layer finish, {T} rows: {us:.1f} us per call ({layer['bf16_mfma_frac']:.3f} of the bf16 MFMA peak); "
        + ", ".join(f"{k} {v['us_avg']:.1f} us" for k, v in layer["kernels"].items()))
    # The same layer on the block's rows only (the deeper layers' approximate
    # step): HBM-bound on the weights, the GEMMs split their contraction.
    Mb = wl.block_size
    wsb = ctx.layer_workspace(F, Mb, True, dev)
    ub, pb = timed_calls(lambda i: ctx.layer_finish(F, sets[i % n_sets], hd[:Mb], od[:Mb], out[:Mb], r_out=r[:Mb],
                                                    workspace=wsb, stream=stream))
    accb = layer_accounting(Mb, D, HD, F)
    bytes_b = sum(a["bytes"] for a in accb.values())
    layer_block = {"rows": Mb, "us_per_call": ub, "hbm_frac": bytes_b / (ub * 1e-6) / 1e9 / HBM_PEAK_GBS,
                   "kernels": _kernel_fracs(accb, pb), "algorithmic_bytes": {k: a["bytes"] for k, a in accb.items()}}
    log(f"[bench] layer finish, {Mb} block rows: {ub:.1f} us per call ({layer_block['hbm_frac']:.3f} of HBM peak); "
        + ", ".join(f"{k} {v['us_avg']:.1f} us" for k, v in layer_block["kernels"].items()))
    layer["block_rows"] = layer_block
    del sets, ws, wsb, r
    lm = synth.lm_head_params(D, V, 0)
    gd, wd = bf(lm["gamma_f"]), bf(lm["w_lm"])
    del lm
    sampler = {"vocab": V, "protocol": "cold (the 1 GB lm-head exceeds the memory-side cache)"}
    for name, table in (("cut", wl.table()), ("uncut", [(off, n, 0, n) for off, n, _, _ in wl.table()])):
        M = sum(be - bs for _, _, bs, be in table)
        token = torch.empty(M, dtype=torch.int32, device=dev)
        conf = torch.empty(M, dtype=torch.float32, device=dev)
        sws = ctx.sampler_workspace(V, table, dev)
        us, prof = timed_calls(lambda i: ctx.sampler_cut(out, table, gd, wd, token, conf, workspace=sws, stream=stream))
        acc = sampler_accounting(M, D, V)
        sampler[name] = {"rows": M, "us_per_call": us, "kernels": _kernel_fracs(acc, prof),
                         "algorithmic_bytes": {k: a["bytes"] for k, a in acc.items()}}
        log(f"[bench] sampler {name}, {M} rows: {us:.1f} us per call; "
            + ", ".join(f"{k} {v['us_avg']:.1f} us" for k, v in sampler[name]["kernels"].items()))
        del sws
    sampler["cut_speedup"] = sampler["uncut"]["us_per_call"] / sampler["cut"]["us_per_call"]
    assert ctx.read_device_status() == 0
    return {"layer0_finish": layer, "sampler": sampler}


def measure_multilayer(dev, n_layers=4, vocab=32768, intervals=(None, 10, 5, 2, 1)):
    """Approximate deeper-layer reuse (exact_attention_state_amd.multilayer) at
    LLaDA-8B's layer shape (d_model 4096, 32 x 128 heads, d_ff 12288; W_qkv ~
    N(0, 0.02^2)) with n_layers layers on llada8b's sequence (768 rows, block
    32): one block of the workload's 20 inner steps with its seeded edits, for
    each refresh interval r (None: block boundary only; 1: the full recompute
    every step).  Per r: the relative error of the block rows' final output
    against the full recompute at every step (mean and max over the steps),
    and the GPU time of the block (event-bracketed, eager launches)."""
    import numpy as np
    import torch
    from exact_attention_state_amd import synth
    from exact_attention_state_amd.multilayer import MultiLayer
    wl = synth.WORKLOADS["llada8b"]
    D, H, dh, F = wl.d_model, wl.n_heads, wl.head_dim, synth.LLADA_D_FF
    p = synth.multilayer_params(D, H, dh, F, n_layers, vocab, qkv_std=0.02)
    table = wl.table()
    rng = np.random.default_rng([synth.BASE_SEED, 7, 7])
    ids = rng.integers(0, vocab, wl.total_tokens).astype(np.int32)
    rows = np.concatenate([np.arange(o + bs, o + be) for o, _, bs, be in table])
    import dataclasses
    wl_v = dataclasses.replace(wl, vocab=vocab)                    # edits draw ids from this vocabulary
    steps = [ids]
    for k in range(1, wl.steps):
        ids, _ = synth.step_ids(wl_v, ids, k)
        steps.append(ids)
    dsteps = [(torch.from_numpy(x).to(dev), torch.from_numpy(x[rows].copy()).to(dev)) for x in steps]
    approx = MultiLayer(p, dh, F, table, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, device=dev)
    exact = MultiLayer(p, dh, F, table, rope_theta=wl.rope_theta, rms_eps=wl.rms_eps, device=dev, weights_from=approx)
    del p
    ref, _ = exact.run_block(dsteps, 1)
    ref = [x.double() for x in ref]
    res = {"shape": {"layers": n_layers, "rows": wl.total_tokens, "block": wl.block_size, "d_model": D,
                     "heads_x_head_dim": H * dh, "d_ff": F, "qkv_std": 0.02, "vocab": vocab},
           "steps": len(steps), "intervals": {}}
    for r in intervals:
        approx.run_block(dsteps[:2], r)                          # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        outs, refreshed = approx.run_block(dsteps, r)
        e1.record()
        torch.cuda.synchronize()
        err = [float(torch.linalg.norm(o.double() - g) / torch.linalg.norm(g)) for o, g in zip(outs, ref)]
        res["intervals"][str(r)] = {"ms_per_block": e0.elapsed_time(e1), "refreshes": int(sum(refreshed)),
                                    "rel_err_mean": float(np.mean(err)), "rel_err_max": float(np.max(err)),
                                    "rel_err_per_step": err}
        log(f"[bench] approximate reuse, {n_layers} layers, r = {r}: {e0.elapsed_time(e1):.2f} ms per block of "
            f"{len(steps)} steps ({sum(refreshed)} refreshes), error vs full recompute mean {np.mean(err):.2e} "
            f"max {np.max(err):.2e}")
    return res


def measure_flashdllm(dev, reps=50, budget=32):
    """The selective cache update and two-view verify on llada8b after a
    block step: lacache_track_select (importance of the 768 rows for the 32
    block queries, then the 32-row tracking set) and lacache_verify_attn with a
    verify query of the tracking set, a 32-token draft view and a 32-token mask
    view (96 tokens) over the cached rows.  Median microseconds per call over
    `reps` calls, and each call's algorithmic bytes (the sample's K rows for
    the importance; K and V rows for the verify attention) against 8 TB/s."""
    import numpy as np
    import torch
    from exact_attention_state_amd import synth
    from exact_attention_state_amd.workload import DeviceWorkload
    wl = synth.WORKLOADS["llada8b"]
    dw = DeviceWorkload(wl, device=dev)
    dw.prefill()
    dw.block_step(dw.next_block_ids())
    torch.cuda.synchronize()
    (off, n, bs, be), = dw.table
    H, Hk, d = wl.n_heads, wl.n_kv_heads, wl.head_dim
    imp = torch.zeros(dw.n_rows, dtype=torch.float32, device=dev)
    trk = torch.empty(1, budget, dtype=torch.int32, device=dev)
    ws = dw.ctx.track_workspace(dw.n_rows, dev)
    rng = np.random.default_rng(5)
    S = be - bs
    others = np.setdiff1d(np.arange(n), np.arange(bs, be))
    pos = np.concatenate([np.sort(rng.choice(others, budget, replace=False)), np.arange(bs, be), np.arange(bs, be)])
    view = np.concatenate([np.zeros(budget), np.ones(S), 2 * np.ones(S)]).astype(np.int32)
    V = len(pos)
    qv, kv, vv = (torch.randn(V, hh, d, device=dev, dtype=torch.float16) for hh in (H, Hk, Hk))
    pos_d, view_d = torch.from_numpy(pos.astype(np.int32)).to(dev), torch.from_numpy(view).to(dev)
    out = torch.empty(V, H, d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(V, H, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[reps // 2]

    t_trk = timed(lambda: dw.ctx.track_select(dw.ct, dw.table, budget, imp, trk, workspace=ws))
    t_ver = timed(lambda: dw.ctx.verify_attn(qv, kv, vv, view_d, pos_d, [0, V], dw.ct, dw.table, out, lse))
    # Kernel time alone (events stamped by the dispatches; the call times above include the host's launch path).
    dw.ctx.profile(True)
    dw.ctx.profile_read()
    for _ in range(reps):
        dw.ctx.track_select(dw.ct, dw.table, budget, imp, trk, workspace=ws)
        dw.ctx.verify_attn(qv, kv, vv, view_d, pos_d, [0, V], dw.ct, dw.table, out, lse)
    torch.cuda.synchronize()
    prof = dw.ctx.profile_read()
    dw.ctx.profile(False)
    kus = {k: prof[k][0] * 1e3 / max(prof[k][1], 1) for k in ("track_importance", "track_select", "verify_attn")}
    kv_row = Hk * d * 2
    b_trk, b_ver = n * kv_row + S * H * d * 2, 2 * n * kv_row + V * (H + 2 * Hk) * d * 2
    k_trk = kus["track_importance"] + kus["track_select"]
    res = {"budget": budget, "verify_tokens": V,
           "track_select": {"us_per_call": t_trk, "kernel_us": {k: kus[k] for k in ("track_importance", "track_select")},
                            "algorithmic_bytes": b_trk, "hbm_frac_kernels": b_trk / (k_trk * 1e-6) / 1e9 / HBM_PEAK_GBS},
           "verify_attn": {"us_per_call": t_ver, "kernel_us": kus["verify_attn"], "algorithmic_bytes": b_ver,
                           "hbm_frac_kernel": b_ver / (kus["verify_attn"] * 1e-6) / 1e9 / HBM_PEAK_GBS}}
    log(f"[bench] selective update: track_select {t_trk:.1f} us per call (kernels: importance "
        f"{kus['track_importance']:.1f} us, selection {kus['track_select']:.1f} us); verify attention ({V} tokens) "
        f"{t_ver:.1f} us per call ({kus['verify_attn']:.1f} us kernel)")
    assert dw.ctx.read_device_status() == 0
    return res


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the layer-0 step is sharded by sample or head in a multi-GPU design; nothing here runs it)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from exact_attention_state_amd import lacache, synth
    from exact_attention_state_amd.workload import DeviceWorkload, to_device_array

    ffn_rows = [int(x) for x in args.ffn_rows.split(",") if x.strip()]
    if args.ffn_only:
        torch.cuda.init()
        print(json.dumps({"ffn_fp8": measure_ffn(torch.device("cuda:0"), ffn_rows)}), flush=True)
        return
    if args.layer_only:
        torch.cuda.init()
        print(json.dumps(measure_layer(torch.device("cuda:0"))), flush=True)
        return
    if args.multilayer_only:
        torch.cuda.init()
        print(json.dumps({"approx_reuse": measure_multilayer(torch.device("cuda:0")),
                          "selective_verify": measure_flashdllm(torch.device("cuda:0"))}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    acc = step_accounting(wl)
    log(f"[bench] workload {wl.name}: batch {wl.batch} N {wl.seq_lens[:4]} block {wl.block_size} "
        f"M {acc['M']} dtype {wl.dtype}")
    torch.cuda.init()
    dev = torch.device("cuda:0")
    t0 = time.time()
    base = DeviceWorkload(wl, device=dev)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")
    ctx = base.ctx
    sets = [base]
    for i in range(1, args.sets):
        # An independent copy of the layer: its own W_qkv, caches and workspace.
        s = DeviceWorkload.__new__(DeviceWorkload)
        s.__dict__.update(base.__dict__)
        w2 = base.weights[2].clone()
        s.weights = (base.weights[0], base.weights[1], w2)
        if len(base.weights) > 3:
            s.weights = s.weights + (ctx.pack_qkv_weight(w2),)
        s.ct = ctx.alloc_cache(base.n_rows, dev)
        s.ws = ctx.alloc_workspace(lacache.OP_BLOCK_STEP, base.table, dev)
        sets.append(s)
    for s in sets:
        s.prefill()
    torch.cuda.synchronize()
    log(f"[bench] {len(sets)} sets prefilled")

    # The 20 seeded edit steps, as device block-id tensors (cycled).
    blk_ids = []
    ids = base.ids_host
    for k in range(1, wl.steps + 1):
        ids, blk = synth.step_ids(wl, ids, k)
        blk_ids.append(torch.from_numpy(blk).to(dev))

    # Prebuilt ctypes arguments per set so the loop is one C call per step.
    lib = ctx.lib
    seqs = lacache._seqs(base.table)
    pre = []
    for s in sets:
        w = ctx._weights(*s.weights)
        c = ctx._cache(s.ct)
        pre.append((w, c, s.ct.out.data_ptr(), s.ct.lse.data_ptr(), s.ws.data_ptr(), s.ws.numel()))
    import ctypes

    def run_step(i, stream_handle, which=None):
        j = i % len(sets) if which is None else which
        w, c, out, lse, ws, wsn = pre[j]
        st = lib.lacache_block_step(ctx.handle, ctypes.byref(w), ctypes.c_void_p(blk_ids[i % len(blk_ids)].data_ptr()),
                                    seqs, len(base.table), ctypes.byref(c), ctypes.c_void_p(out),
                                    ctypes.c_void_p(lse), ctypes.c_void_p(ws), wsn, stream_handle)
        if st != 0:
            raise RuntimeError(lib.lacache_last_error(ctx.handle).decode())

    stream = torch.cuda.Stream(device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def timed_eager(K, which=None):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            run_step(i, sh, which)
        stream.synchronize()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    # Warm-up (eager) and the eager timing.
    for i in range(args.warmup):
        run_step(i, sh)
    stream.synchronize()
    ms_eager = timed_eager(args.steps)
    log(f"[bench] eager: {ms_eager * 1e3:.2f} us/step")

    # HIP graph of one cycle of steps over the rotating sets, replayed.
    ms_graph = None
    graph_err = None
    if not args.no_graph:
        try:
            cyc = len(blk_ids)      # one cycle of the seeded edits (a multiple of the set count)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                with torch.cuda.graph(g, stream=stream):
                    for i in range(cyc):
                        run_step(i, ctypes.c_void_p(stream.cuda_stream))
            reps = max(1, -(-args.steps // cyc))
            for _ in range(max(1, args.warmup // cyc)):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            graph_steps = reps * cyc
            ms_graph = (time.perf_counter() - t0) * 1e3 / graph_steps
            log(f"[bench] hip graph: {ms_graph * 1e3:.2f} us/step ({reps} x {cyc} steps)")
        except Exception as e:  # graph capture is an optimisation of the launch path only
            graph_err = repr(e)
            log(f"[bench] graph capture unavailable: {graph_err}")

    # Warm (single set) eager timing, context only.
    ms_warm = timed_eager(args.steps, which=0)
    log(f"[bench] warm (one set, eager): {ms_warm * 1e3:.2f} us/step")

    # Per-kernel durations: a separate eager pass with every launch bracketed by
    # events on the launch stream.  A bounded matmul queued first keeps the GPU
    # busy while the host enqueues all steps, so the events bracket back-to-back
    # GPU execution rather than host submission gaps.
    ctx.profile(True)
    ctx.profile_read()
    torch.cuda.synchronize()
    big = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        for _ in range(8):
            big = (big @ big).clamp_(-1, 1)
    for i in range(args.steps):
        run_step(i, sh)
    stream.synchronize()
    torch.cuda.synchronize()
    prof = ctx.profile_read()
    ctx.profile(False)
    del big
    kern = {k: {"ms_total": v[0], "launches": v[1], "us_avg": (v[0] * 1e3 / v[1]) if v[1] else None}
            for k, v in prof.items() if v[1]}
    log(f"[bench] per-kernel: " + ", ".join(f"{k} {v['us_avg']:.2f} us" for k, v in kern.items()))

    # Per-step distribution: every step bracketed by events on the launch
    # stream, enqueued behind a bounded matmul as above (GPU time of each step,
    # host submission excluded).
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    big = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        for _ in range(8):
            big = (big @ big).clamp_(-1, 1)
        for i in range(args.steps):
            step_ev[i][0].record(stream)
            run_step(i, sh)
            step_ev[i][1].record(stream)
    torch.cuda.synchronize()
    del big
    per_step = sorted(a.elapsed_time(b) * 1e3 for a, b in step_ev)

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]

    step_pct = {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9), "steps": len(per_step)}
    log(f"[bench] per step (events, eager): p10 {step_pct['p10']:.2f} us, median {step_pct['median']:.2f} us, "
        f"p90 {step_pct['p90']:.2f} us")

    refresh = (measure_refresh(ctx, sets, base, stream, dev, args.refresh_reps, acc, wl, blk_ids[0])
               if args.refresh_reps > 0 else None)

    # Parity is the tests' job; here the outputs must be finite and the device
    # status word clear (no q/k/v value beyond the fp16 range, no bad id).
    assert torch.isfinite(base.ct.out.float()).all()
    device_status = ctx.read_device_status()
    if device_status:
        raise RuntimeError(f"device status flags {device_status:#x} after the timed steps")

    ms = ms_graph if ms_graph is not None else ms_eager
    steps_timed = graph_steps if ms_graph is not None else args.steps
    if refresh is not None:
        # One block: its refresh at the boundary, then the workload's inner steps.
        refresh["us_per_step_amortized"] = (refresh["us_per_block_refresh"] + wl.steps * ms * 1e3) / (wl.steps + 1)
        refresh["us_per_step_amortized_full_refresh"] = (refresh["us_per_refresh"] + wl.steps * ms * 1e3) / (wl.steps + 1)
    value = acc["pairs_computed"] / (ms * 1e-3)

    # Roofline of the dominant kernel.
    dom = max((k for k in kern if k in acc["kernels"]), key=lambda k: kern[k]["ms_total"])
    t_dom = kern[dom]["us_avg"] * 1e-6
    flops, nbytes = acc["kernels"][dom]["flops"], acc["kernels"][dom]["bytes"]
    peak_flops = (MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS) * 1e12
    ridge = peak_flops / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes < ridge:
        roof = {"bound": "hbm", "achieved": nbytes / t_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": peak_flops / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["bound"] == "hbm":
        # Beside the nominal peak: the fraction of what a plain device copy reaches.
        roof["stream_copy_GBps"] = stream_copy_gbs(dev)
        roof["frac_of_copy"] = roof["achieved"] / roof["stream_copy_GBps"]
    roof["traffic"] = measured_traffic(dom, wl.name)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = nbytes
    roof["flops"] = flops

    ffn = measure_ffn(dev, ffn_rows) if ffn_rows else None
    layer = None if args.no_layer else measure_layer(dev)
    approx_reuse = None if args.no_multilayer else measure_multilayer(dev)
    sel_verify = None if args.no_flashdllm else measure_flashdllm(dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] oracle CPU baseline ...")
        cpu = cpu_baseline(wl, args.cpu_seconds, ms * 1e-3)
        log(f"[bench] oracle: full recompute {cpu['s_per_step_full_recompute']:.3f} s "
            f"({cpu['ratio_to_gpu_step']:.0f} x the GPU step), cached step {cpu['cached_step']['ms_per_step']:.1f} ms, "
            f"{cpu['cores']} threads on {cpu['host']['cpu_model']}")

    line = {
        "metric": "query-key pairs/s of the exact LaCache layer-0 cached block step (LLaDA-8B layer 0)",
        "value": value,
        "unit": "query-key pairs/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": ms * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian parameters, uniform token ids)",
        "arithmetic": ({"parameters": "bf16", "matrix_core_operands": "fp16 (bf16 weights converted exactly; "
                        "gamma*E rounded to fp16 once)", "accumulation": "fp32", "softmax": "fp32",
                        "caches": "fp16 RoPECache q/k/v and FACache O~/l; fp32 FACache m, l", "output": "bf16, LSE fp32"}
                       if wl.dtype == "bf16" else {"everything": "fp32"}),
        "device_status": device_status,
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_lens[0], "prompt": wl.prompt_lens[0],
                   "block_size": wl.block_size, "d_model": wl.d_model, "heads": wl.n_heads,
                   "head_dim": wl.head_dim, "vocab": wl.vocab, "cache_protocol": f"cold ({len(sets)} rotating sets)",
                   "launch": "hipgraph" if ms_graph is not None else "eager"},
        "pairs_computed_per_step": acc["pairs_computed"],
        "pairs_equiv_per_s": acc["pairs_equiv"] / (ms * 1e-3),
        "us_per_step_eager": ms_eager * 1e3,
        "us_per_step_events": step_pct,
        "us_per_step_graph": None if ms_graph is None else ms_graph * 1e3,
        "us_per_step_warm_eager": ms_warm * 1e3,
        "kernels_us_avg": {k: v["us_avg"] for k, v in kern.items()},
        "kernels_hbm_frac": {k: acc["kernels"][k]["bytes"] / (v["us_avg"] * 1e-6) / 1e9 / HBM_PEAK_GBS
                             for k, v in kern.items() if k in acc["kernels"]},
        "kernels_mfma_frac": {k: acc["kernels"][k]["flops"] / (v["us_avg"] * 1e-6) / peak_flops
                              for k, v in kern.items() if k in acc["kernels"] and acc["kernels"][k]["flops"]},
        "kernel_source_sha256": {k: kernel_source_hash(k) for k in kern},
        "attention": attention_summary(acc, kern),
        "projection": projection_summary(acc, kern, peak_flops),
        "roofline": roof,
        "refresh": refresh,
        "ffn_fp8": ffn,
        "layer0_finish": None if layer is None else layer["layer0_finish"],
        "sampler": None if layer is None else layer["sampler"],
        "approx_reuse": approx_reuse,
        "selective_verify": sel_verify,
        "cpu_baseline": cpu,
        "host": platform.node(),
        "graph_error": graph_err,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
