"""Plain CPU oracle of LaCache's per-group FP8 FFN (layers after the first).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes (LaCache, "Exact Caching and Precision-Adaptive Inference
for Diffusion Large Language Models", arXiv 2607.16339, Section 3.4 "Mixed
precision strategy", Eqs. (7)-(8), and Figure 2):

* Per-group quantization: a tensor is split into groups g; each group gets
  ``scale_g = max_{i in g} |x_i| / Q_max`` (Eq. (8)) and its elements become
  ``x'_i = clip(x_i / scale_g, Q_min, Q_max)`` in the low-precision format
  (Eq. (7)).  Groups: 1 x 128 on activations (128 consecutive features of one
  token), 128 x 128 on weights.
* The FFN of a layer after the first: AddNorm (the residual add, then the
  feed-forward RMSNorm), quantization fused with it, the gate-up linear on
  the quantized operands, SwiGLU with the quantization of its output fused,
  the ffout (down) linear on the quantized operands, and the residual add.
  The first layer keeps its original precision (Section 3.4).

Readings where the pages are silent (each listed in the design doc):
* Format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
  no infinities, the all-ones code is NaN), the FP8 format the gfx950 matrix
  cores take; Q_max = 448, Q_min = -448.
* Rounding to the format after the clip: round to nearest, ties to even.
* The quantization decision (scale and x / scale) is taken in fp32, the
  precision of the kernels: both the GPU and this oracle compute
  ``scale = fp32(amax) / 448`` and ``fp32(x) / scale`` with correctly rounded
  fp32 division.  A group whose elements are all zero gets scale 0 and codes 0.
* The residual stream is bf16: ``r = bf16(h + attn_out)`` (the exact sum
  rounded to nearest even); the RMSNorm reads r.  The FFN output is
  ``bf16(r + down)``.
* SwiGLU: ``silu(gate) * up`` with ``silu(x) = x / (1 + exp(-x))``; gate and
  up are the two halves of the gate-up linear's output.
Everything else is fp64.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GROUP = 128

__all__ = [
    "E4M3_MAX", "GROUP", "e4m3_values", "e4m3_decode", "round_e4m3", "encode_e4m3", "round_bf16",
    "quantize_activation", "quantize_weight", "dequantize_activation", "dequantize_weight", "fp8_linear",
    "add_norm", "silu", "swiglu", "ffn_fp8", "ffn_exact",
]


# ----------------------------------------------------------------------------
# The E4M3 format
# ----------------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    """Value of an 8-bit E4M3 code: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m * 2^-9); exponent 15 with
    mantissa 7 is NaN (no infinities)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_values() -> np.ndarray:
    """Every finite E4M3 value, sorted (+0 and -0 both appear as 0)."""
    v = np.array([e4m3_decode(c) for c in range(256)])
    return np.unique(v[np.isfinite(v)])


_POS = np.array([e4m3_decode(c) for c in range(0x7F)])       # codes 0..126: +0 .. 448, increasing


def round_e4m3(v) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code (|v| <= 448)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX):
        raise ValueError("round_e4m3 expects |v| <= 448 (clip first)")
    hi = np.searchsorted(_POS, a, side="left")                # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))      # tie: the even code
    q = np.where(a == _POS[hi], _POS[hi], np.where(pick_hi, _POS[hi], _POS[lo]))
    return np.copysign(q, v)


def encode_e4m3(q) -> np.ndarray:
    """The uint8 codes of E4M3 values q (as produced by round_e4m3); +0 for zeros."""
    q = np.asarray(q, np.float64)
    idx = np.searchsorted(_POS, np.abs(q))
    if not np.array_equal(_POS[np.minimum(idx, len(_POS) - 1)], np.abs(q)):
        raise ValueError("not E4M3 values")
    return (idx.astype(np.uint8) | np.where(np.signbit(q) & (q != 0), 0x80, 0).astype(np.uint8))


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (8 significant bits), ties to
    even, returned as fp64.  |x| in [2^(E-1), 2^E) has the bf16 spacing
    2^(E-8); x / spacing is exact, and np.round rounds halves to even."""
    x = np.asarray(x, np.float64)
    _, E = np.frexp(x)
    E = np.maximum(E, -125)                        # below the normal range the spacing stays 2^-133
    ulp = np.ldexp(1.0, E - 8)
    return np.round(x / ulp) * ulp


# ----------------------------------------------------------------------------
# Per-group quantization, Eqs. (7)-(8)
# ----------------------------------------------------------------------------

def _quantize_group_values(x32: np.ndarray, amax32: np.ndarray):
    """Codes of fp32 values x32 with their groups' fp32 maxima (broadcast).

    scale = amax / Q_max and v = x / scale in fp32 (correctly rounded
    division), then clip to [Q_min, Q_max] (Eq. (7)) and round to E4M3."""
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = (amax32 / np.float32(E4M3_MAX)).astype(np.float32)
        v = (x32 / scale).astype(np.float32)
    v = np.where(scale == 0, np.float32(0), v)
    v = np.clip(v.astype(np.float64), -E4M3_MAX, E4M3_MAX)
    return round_e4m3(v), scale


def quantize_activation(x, group: int = GROUP):
    """1 x group quantization of activations x [T, K] (K a multiple of group).

    Returns (q [T, K] E4M3 values, scale [T, K / group] fp32 as fp64)."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    T, K = x32.shape
    g = x32.reshape(T, K // group, group)
    amax = np.max(np.abs(g), axis=2, keepdims=True)
    q, scale = _quantize_group_values(g, amax)
    return q.reshape(T, K), scale[..., 0].astype(np.float64)


def quantize_weight(w, group: int = GROUP):
    """group x group block quantization of a weight w [N, K] (both multiples of group).

    Returns (q [N, K] E4M3 values, scale [N / group, K / group] fp32 as fp64)."""
    w32 = np.asarray(w, np.float64).astype(np.float32)
    N, K = w32.shape
    b = w32.reshape(N // group, group, K // group, group)
    amax = np.max(np.abs(b), axis=(1, 3), keepdims=True)
    q, scale = _quantize_group_values(b, amax)
    return q.reshape(N, K), scale[:, 0, :, 0].astype(np.float64)


def dequantize_activation(q, scale, group: int = GROUP):
    return np.asarray(q, np.float64) * np.repeat(np.asarray(scale, np.float64), group, axis=1)


def dequantize_weight(q, scale, group: int = GROUP):
    s = np.repeat(np.repeat(np.asarray(scale, np.float64), group, axis=0), group, axis=1)
    return np.asarray(q, np.float64) * s


def fp8_linear(qa, sa, qw, sw, group: int = GROUP):
    """y = A W^T on the quantized operands: the dequantized product
    sum_g sa[m, g] sw[n / group, g] sum_{k in g} qa[m, k] qw[n, k], in fp64."""
    return dequantize_activation(qa, sa, group) @ dequantize_weight(qw, sw, group).T


# ----------------------------------------------------------------------------
# The FFN of a layer after the first (Figure 2; Section 3.4)
# ----------------------------------------------------------------------------

def add_norm(h, a, gamma, eps: float):
    """AddNorm: r = bf16(h + a) (the residual stream), x = gamma * r / sqrt(mean(r^2) + eps)."""
    r = round_bf16(np.asarray(h, np.float64) + np.asarray(a, np.float64))
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return r, np.asarray(gamma, np.float64) * r / np.sqrt(ms + eps)


def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu(gate, up):
    return silu(gate) * np.asarray(up, np.float64)


def ffn_fp8(h, a, gamma, w_gate, w_up, w_down, eps: float, group: int = GROUP) -> dict:
    """The per-group FP8 FFN, plainly, step by step.

    h, a [T, D] (bf16 values), gamma [D], w_gate, w_up [F, D], w_down [D, F].
    Returns every intermediate: r, x, (qx, sx), (qgu, sgu) of [w_gate; w_up],
    gate, up, y = swiglu, (qy, sy), (qd, sd), down, out = bf16(r + down)."""
    r, x = add_norm(h, a, gamma, eps)
    qx, sx = quantize_activation(x, group)
    w_gu = np.concatenate([np.asarray(w_gate, np.float64), np.asarray(w_up, np.float64)], axis=0)
    qgu, sgu = quantize_weight(w_gu, group)
    gu = fp8_linear(qx, sx, qgu, sgu, group)
    F = np.shape(w_gate)[0]
    gate, up = gu[:, :F], gu[:, F:]
    y = swiglu(gate, up)
    qy, sy = quantize_activation(y, group)
    qd, sd = quantize_weight(w_down, group)
    down = fp8_linear(qy, sy, qd, sd, group)
    out = round_bf16(r + down)
    return dict(r=r, x=x, qx=qx, sx=sx, qgu=qgu, sgu=sgu, gate=gate, up=up, y=y, qy=qy, sy=sy, qd=qd, sd=sd,
                down=down, out=out)


def ffn_exact(h, a, gamma, w_gate, w_up, w_down, eps: float) -> dict:
    """The same FFN without quantization (fp64 throughout): the reference the
    quantized FFN approximates."""
    r, x = add_norm(h, a, gamma, eps)
    y = swiglu(x @ np.asarray(w_gate, np.float64).T, x @ np.asarray(w_up, np.float64).T)
    down = y @ np.asarray(w_down, np.float64).T
    return dict(r=r, x=x, y=y, down=down, out=r + down)
