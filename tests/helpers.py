"""Shared test helpers: tolerances and comparisons against the fp64 oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle import Layer0Config

# Output tolerances.  fp32 workloads: max |err| <= 1e-5.  bf16 workloads:
# max |err| <= 2e-2 and, per (row, head), the relative error of the output
# row norm | ||o|| - ||o_ref|| | / ||o_ref|| <= 5e-3.
F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_ROWNORM_RTOL = 5e-3
# Intermediate caches (q, k, v, the FACache pair) in bf16 are compared with
# |err| <= BF16_CACHE_ATOL + BF16_CACHE_RTOL |ref| (one bf16 rounding of a
# value that itself carries the rounding of its bf16 inputs).
BF16_CACHE_ATOL = 2e-2
BF16_CACHE_RTOL = 1e-2


def cfg_of(wl) -> Layer0Config:
    return Layer0Config(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.rope_theta, wl.rms_eps)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_output(got, want, dtype, what=""):
    """Compare attention outputs [R, H, d] (or [R, d]) at the output bar.  Returns error stats."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    stats = {"max_abs": float(err.max())}
    nref = np.linalg.norm(want, axis=-1)
    ngot = np.linalg.norm(got, axis=-1)
    stats["rownorm_rel"] = float(np.max(np.abs(ngot - nref) / np.maximum(nref, 1e-30)))
    stats["row_rel"] = float(np.max(np.linalg.norm(got - want, axis=-1) / np.maximum(nref, 1e-30)))
    if dtype == "f32":
        assert stats["max_abs"] <= F32_ATOL, f"{what}: {stats}"
    else:
        assert stats["max_abs"] <= BF16_ATOL, f"{what}: {stats}"
        assert stats["rownorm_rel"] <= BF16_ROWNORM_RTOL, f"{what}: {stats}"
    return stats


def check_lse(got, want, dtype, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite lse"
    e = float(np.max(np.abs(got - want)))
    assert e <= (F32_ATOL if dtype == "f32" else BF16_ATOL), f"{what}: lse max abs err {e}"
    return e


def check_cache_values(got, want, dtype, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    if dtype == "f32":
        e = float(np.max(np.abs(got - want)))
        assert e <= F32_ATOL, f"{what}: max abs err {e}"
    else:
        bound = BF16_CACHE_ATOL + BF16_CACHE_RTOL * np.abs(want)
        bad = np.abs(got - want) > bound
        assert not bad.any(), f"{what}: {int(bad.sum())} values out of tolerance, worst {float(np.max(np.abs(got - want)))}"
