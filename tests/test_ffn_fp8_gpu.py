"""GPU parity of the per-group FP8 FFN (lacache_ffn_pack_weights, lacache_ffn_fp8)
with the FP8 oracle (oracle/fp8_ref.py), stage by stage.

* Weight quantization: every code and every block scale bit-exact (both sides
  divide the same bf16 values by the same fp32 scale, correctly rounded).
* AddNorm: the residual r bit-exact; the codes of x = RMSNorm(r): equal to the
  oracle's wherever the oracle's x / scale is farther from a rounding boundary
  than the GPU's fp32 RMSNorm can move it, else one of the two neighbouring
  codes; scales within the same bound.
* Gate-up + SwiGLU: from the GPU's own x codes and scales, the oracle computes
  gate and up in fp64; the GPU's y codes must be the oracle's rounding of
  y / scale within the error bound of the FP8 GEMM (per 128-wide group
  2^-10 sum |a_k b_k| for the matrix core's internal sum, measured at most
  2^-12.4, plus fp32 accumulation over the groups) carried through SwiGLU.
* Down + residual: from the GPU's own y codes and scales, out must equal
  bf16(r + down) within one bf16 rounding plus the GEMM bound.
* End to end against the oracle's own chain (its own quantization of every
  stage): reported, and bounded at the row-norm level.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import fp8_ref as q8
from exact_attention_state_amd import lacache, synth

pytestmark = pytest.mark.gpu

_DEC = np.array([q8.e4m3_decode(c) for c in range(256)])
GEMM_REL = 2.0 ** -10           # the matrix core's internal sum, per 128-wide group (measured <= 2^-12.4)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def unpack(packed: np.ndarray, n_rows: int, K: int) -> np.ndarray:
    """Values [n_rows, K] of a packed FP8 operand (the layout documented in include/lacache.h)."""
    Np = -(-n_rows // 256) * 256
    b = np.asarray(packed, np.uint8)[: Np * K].reshape(Np // 256, K // 128, 16, 2, 4, 16, 16)
    # axes: tile, group, 16-row fragment, half, lane group, row in fragment, byte
    b = b.transpose(0, 2, 5, 1, 4, 3, 6).reshape(Np, K)
    return _DEC[b[:n_rows]]


def _ctx(D, F):
    return lacache.Context(D, D // 128, D // 128, 128, 1000, 64, 1e4, 1e-5, 0.0, "bf16")


def _bf16(x, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(dev)


def _run(D, F, T, seed, family=0):
    ctx = _ctx(D, F)
    p = synth.ffn_params(D, F, family)
    h, a = synth.ffn_inputs(T, D, seed)
    wg, wu, wd, g = (_bf16(p[k]) for k in ("w_gate", "w_up", "w_down", "gamma"))
    packed = ctx.ffn_pack_weights(F, wg, wu, wd)
    hd, ad = _bf16(h), _bf16(a)
    out = torch.empty_like(hd)
    r = torch.empty_like(hd)
    ws = ctx.ffn_fp8(F, g, packed, hd, ad, out, r_out=r)
    torch.cuda.synchronize()
    return ctx, p, h, a, packed, ws, r, out


def _workspace(ws, T, D, F):
    """The workspace parts after the call (layout documented in include/lacache.h)."""
    Mp = -(-T // 256) * 256
    al = lambda x: -(-x // 256) * 256
    raw = ws.cpu().numpy()
    o = 0
    parts = {}
    for name, nbytes in (("xq", Mp * D), ("sx", D // 128 * Mp * 4), ("yq", Mp * F), ("sy", F // 128 * Mp * 4)):
        parts[name] = raw[o:o + nbytes]
        o += al(nbytes)
    qx = unpack(parts["xq"], T, D)
    sx = parts["sx"].view(np.float32).reshape(D // 128, Mp)[:, :T].T.astype(np.float64)
    qy = unpack(parts["yq"], T, F)
    sy = parts["sy"].view(np.float32).reshape(F // 128, Mp)[:, :T].T.astype(np.float64)
    return qx, sx, qy, sy


def _packed_weights(packed, D, F):
    gu, sgu, dn, sdn = (t.cpu().numpy() for t in packed)
    qgu_p = unpack(gu, 2 * F, D)                        # rows: tile j = [gate 128 j.., up 128 j..]
    j = np.arange(2 * F)
    tile, c = j // 256, j % 256
    src = np.where(c < 128, 128 * tile + c, F + 128 * tile + c - 128)
    qgu = np.empty_like(qgu_p)
    qgu[src] = qgu_p                                   # rows of [w_gate; w_up]
    s = sgu.reshape(D // 128, 2 * F // 128)            # [group][packed block]
    blk = np.arange(2 * F // 128)
    src_b = np.where(blk % 2 == 0, blk // 2, F // 128 + blk // 2)
    sgu_rows = np.empty((2 * F // 128, D // 128))
    sgu_rows[src_b] = s.T
    qd = unpack(dn, D, F)
    sd = sdn.reshape(F // 128, D // 128).T.astype(np.float64)
    return qgu, sgu_rows, qd, sd


def _code_window(v, tol):
    """E4M3 values that rounding any value within v +- tol can give (lowest, highest)."""
    lo = q8.round_e4m3(np.clip(v - tol, -448, 448))
    hi = q8.round_e4m3(np.clip(v + tol, -448, 448))
    return lo, hi


def _check_codes(what, q_gpu, s_gpu, ref, ref_err):
    """GPU codes q_gpu (values) with scales s_gpu [T, groups] against the
    oracle's values ref whose GPU counterpart may differ by ref_err."""
    T, K = ref.shape
    amax_ref = np.abs(ref).reshape(T, K // 128, 128).max(axis=2)
    err_max = ref_err.reshape(T, K // 128, 128).max(axis=2)
    assert np.all(np.abs(s_gpu * 448 - amax_ref) <= err_max * (1 + 1e-6) + amax_ref * 2.0 ** -22), f"{what}: scales"
    sc = np.repeat(s_gpu, 128, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(sc > 0, ref / sc, 0.0)
        tol = np.where(sc > 0, ref_err / sc + np.abs(v) * 2.0 ** -22, 0.0)
    lo, hi = _code_window(v, tol)
    ok = (q_gpu >= lo) & (q_gpu <= hi)
    assert ok.all(), f"{what}: {int((~ok).sum())} codes outside their window, e.g. {np.argwhere(~ok)[:3].tolist()}"
    ambiguous = float(np.mean(lo != hi))
    exact = float(np.mean(q_gpu == q8.round_e4m3(np.clip(v, -448, 448))))
    return {"codes": q_gpu.size, "ambiguous_frac": ambiguous, "equal_to_oracle_frac": exact}


def _gemm_bound(qa, sa, qw, sw):
    """|A W^T| error bound of the FP8 GEMM on these operands."""
    KG = qa.shape[1] // 128
    absprod = q8.fp8_linear(np.abs(qa), sa, np.abs(qw), sw)
    return (GEMM_REL + KG * 2.0 ** -23) * absprod


# (512, 6144, 301): the down projection's 16 tiles of 128 x 128 contract over
# 48 groups and split in two (partials summed by a second kernel).
@pytest.mark.parametrize("D,F,T", [(512, 384, 77), (1024, 768, 300), (512, 1024, 513), (512, 6144, 301)])
def test_ffn_fp8_every_stage(D, F, T, monkeypatch):
    _say(f"[ffn] D {D} F {F} T {T}")
    if T == 300:
        monkeypatch.setenv("LACACHE_FP8_TILE", "256")           # the 256 x 256 down tile on a small launch
    ctx, p, h, a, packed, ws, r, out = _run(D, F, T, seed=T)
    eps = 1e-5
    # weights: bit-exact codes and scales
    qgu, sgu, qd, sd = _packed_weights(packed, D, F)
    w_gu = np.concatenate([p["w_gate"], p["w_up"]], axis=0)
    qgu_ref, sgu_ref = q8.quantize_weight(w_gu)
    qd_ref, sd_ref = q8.quantize_weight(p["w_down"])
    assert np.array_equal(qgu, qgu_ref) and np.array_equal(sgu, sgu_ref), "gate-up weight codes/scales"
    assert np.array_equal(qd, qd_ref) and np.array_equal(sd, sd_ref), "down weight codes/scales"
    # AddNorm: r bit-exact, x codes within their windows
    r_ref, x_ref = q8.add_norm(h, a, p["gamma"], eps)
    assert np.array_equal(r.float().cpu().numpy().astype(np.float64), r_ref), "residual r"
    qx, sx, qy, sy = _workspace(ws, T, D, F)
    x_err = np.abs(x_ref) * 2.0 ** -16                       # fp32 RMSNorm: the sum of squares over d_model
    st_x = _check_codes("x codes", qx, sx, x_ref, x_err)
    # gate-up + SwiGLU from the GPU's own x
    gu = q8.fp8_linear(qx, sx, qgu, sgu)
    gu_err = _gemm_bound(qx, sx, qgu, sgu)
    gate, up = gu[:, :F], gu[:, F:]
    y_ref = q8.swiglu(gate, up)
    e_g, e_u = gu_err[:, :F], gu_err[:, F:]
    sig = 1 / (1 + np.exp(-gate))
    dsilu = sig * (1 + gate * (1 - sig))                      # d silu / d gate, |.| <= 1.1
    y_err = (np.abs(dsilu * up) + 1.1 * e_u) * e_g + np.abs(q8.silu(gate)) * e_u + np.abs(y_ref) * 2.0 ** -19
    st_y = _check_codes("y codes", qy, sy, y_ref, y_err)
    # down + residual from the GPU's own y
    down = q8.fp8_linear(qy, sy, qd, sd)
    d_err = _gemm_bound(qy, sy, qd, sd)
    got = out.float().cpu().numpy().astype(np.float64)
    pre = r_ref + down
    tol = 2.0 ** -8 * (np.abs(pre) + d_err) + d_err * (1 + 2.0 ** -8) + np.abs(pre) * 2.0 ** -23
    bad = np.abs(got - pre) > tol
    assert not bad.any(), f"out: {int(bad.sum())} values beyond the bound; worst {float(np.max(np.abs(got - pre) - tol))}"
    # end to end against the oracle's own chain
    ref = q8.ffn_fp8(h, a, p["gamma"], p["w_gate"], p["w_up"], p["w_down"], eps)
    rel = np.linalg.norm(got - ref["out"], axis=1) / np.linalg.norm(ref["out"], axis=1)
    _say(f"[ffn] x {st_x} y {st_y}; out vs the oracle's own chain: row rel max {rel.max():.2e}")
    assert rel.max() < 5e-3
    # The windows allow a neighbouring code wherever the GPU's error bound
    # reaches a rounding boundary; the GPU's actual errors are far smaller, so
    # nearly every code must be the oracle's own (a misplaced feature, scale
    # or group would make most of them differ).
    assert st_x["equal_to_oracle_frac"] > 0.999 and st_y["equal_to_oracle_frac"] > 0.99
    assert ctx.read_device_status() == 0


def test_ffn_fp8_llada8b_sampled_rows():
    """LLaDA-8B's FFN shape (d_model 4096, d_ff 12288) on the 768 rows of the
    llada8b sequence: weights bit-exact in full, and 12 sampled rows through
    every stage against the oracle (the 128 x 128 down tile)."""
    D, F, T = 4096, synth.LLADA_D_FF, 768
    _say(f"[ffn] llada8b shape: D {D} F {F} T {T}")
    ctx, p, h, a, packed, ws, r, out = _run(D, F, T, seed=2, family=2)
    qgu, sgu, qd, sd = _packed_weights(packed, D, F)
    qgu_ref, sgu_ref = q8.quantize_weight(np.concatenate([p["w_gate"], p["w_up"]], axis=0))
    assert np.array_equal(qgu, qgu_ref) and np.array_equal(sgu, sgu_ref), "gate-up weight"
    del qgu_ref
    qd_ref, sd_ref = q8.quantize_weight(p["w_down"])
    assert np.array_equal(qd, qd_ref) and np.array_equal(sd, sd_ref), "down weight"
    rng = np.random.default_rng([20261202, 4096])
    rows = np.sort(rng.choice(T, size=12, replace=False))
    r_ref, x_ref = q8.add_norm(h[rows], a[rows], p["gamma"], 1e-5)
    assert np.array_equal(r.float().cpu().numpy()[rows].astype(np.float64), r_ref)
    qx, sx, qy, sy = _workspace(ws, T, D, F)
    st_x = _check_codes("x codes", qx[rows], sx[rows], x_ref, np.abs(x_ref) * 2.0 ** -16)
    gu = q8.fp8_linear(qx[rows], sx[rows], qgu, sgu)
    gu_err = _gemm_bound(qx[rows], sx[rows], qgu, sgu)
    gate, up = gu[:, :F], gu[:, F:]
    y_ref = q8.swiglu(gate, up)
    sig = 1 / (1 + np.exp(-gate))
    dsilu = sig * (1 + gate * (1 - sig))
    e_g, e_u = gu_err[:, :F], gu_err[:, F:]
    y_err = (np.abs(dsilu * up) + 1.1 * e_u) * e_g + np.abs(q8.silu(gate)) * e_u + np.abs(y_ref) * 2.0 ** -19
    st_y = _check_codes("y codes", qy[rows], sy[rows], y_ref, y_err)
    down = q8.fp8_linear(qy[rows], sy[rows], qd, sd)
    d_err = _gemm_bound(qy[rows], sy[rows], qd, sd)
    got = out.float().cpu().numpy()[rows].astype(np.float64)
    pre = r_ref + down
    tol = 2.0 ** -8 * (np.abs(pre) + d_err) + d_err * (1 + 2.0 ** -8) + np.abs(pre) * 2.0 ** -23
    assert not (np.abs(got - pre) > tol).any(), "out beyond the bound"
    _say(f"[ffn] llada8b rows {rows.tolist()}: x {st_x} y {st_y}")
    assert st_x["equal_to_oracle_frac"] > 0.999 and st_y["equal_to_oracle_frac"] > 0.99
    assert ctx.read_device_status() == 0


def test_ffn_fp8_rejects_bad_arguments():
    ctx = _ctx(512, 384)
    with pytest.raises(lacache.LaCacheError) as ei:
        ctx.ffn_workspace(100, 10)                              # d_ff not a multiple of 128
    assert ei.value.status == lacache.ERR_UNSUPPORTED
    p = synth.ffn_params(512, 384)
    packed = ctx.ffn_pack_weights(384, *(_bf16(p[k]) for k in ("w_gate", "w_up", "w_down")))
    h = torch.zeros(8, 512, dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(h, 3.0)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(lacache.LaCacheError) as ei:
        ctx.ffn_fp8(384, _bf16(p["gamma"]), packed, h, h, out, r_out=None, workspace=small)
    assert ei.value.status == lacache.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
