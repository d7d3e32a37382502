"""Pins of the FP8 FFN oracle (oracle/fp8_ref.py) against things other than itself.

The E4M3 format against its definition's fixed points and torch's
float8_e4m3fn cast; bf16 rounding against torch's cast; the per-group
quantization of Eqs. (7)-(8) against closed forms (group maxima land on
Q_max, power-of-two invariance, independence of groups, the format's error
bound); the quantized linear against torch matmul and against exact products
of grid-representable operands; AddNorm and SwiGLU against torch; and the
whole FFN against the unquantized FFN.  No GPU is used.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import fp8_ref as q8


def _rng(*s):
    return np.random.default_rng([8, *s])


# -------------------------------------------------------------- the format ---

def test_e4m3_fixed_points_of_the_definition():
    vals = q8.e4m3_values()
    assert len(vals) == 253                       # 256 codes - 2 NaNs - the duplicate zero
    assert vals.max() == 448.0 and vals.min() == -448.0
    assert q8.e4m3_decode(0x7E) == 448.0          # largest finite: 1.75 * 2^8
    assert math.isnan(q8.e4m3_decode(0x7F)) and math.isnan(q8.e4m3_decode(0xFF))
    assert q8.e4m3_decode(0x38) == 1.0
    assert q8.e4m3_decode(0x08) == 2.0 ** -6      # smallest normal
    assert q8.e4m3_decode(0x01) == 2.0 ** -9      # smallest subnormal
    assert q8.e4m3_decode(0x80) == 0.0 and math.copysign(1, q8.e4m3_decode(0x80)) < 0
    # 8 values per binade above the subnormals: the spacing is 2^(e-3)
    pos = vals[vals >= 2.0 ** -6]
    for e in range(-6, 8):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(b) == 8 and np.allclose(np.diff(b), 2.0 ** (e - 3))


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([q8.e4m3_decode(c) for c in range(256)])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(ref[~both_nan], got[~both_nan]) and np.array_equal(np.isnan(ref), np.isnan(got))


def test_round_e4m3_matches_torch_cast():
    r = _rng(1)
    # fp32 values across every binade of the format, and every midpoint (ties).
    x = (r.standard_normal(20000) * np.exp2(r.integers(-12, 9, size=20000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    vals = q8.e4m3_values()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, vals.astype(np.float32)]).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = q8.round_e4m3(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


def test_encode_decode_round_trip():
    vals = q8.e4m3_values()
    codes = q8.encode_e4m3(vals)
    assert np.array_equal([q8.e4m3_decode(int(c)) for c in codes], vals)


def test_round_bf16_matches_torch_cast():
    r = _rng(2)
    x = (r.standard_normal(20000) * np.exp2(r.integers(-20, 20, size=20000))).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(q8.round_bf16(x), ref)


# ------------------------------------------------- quantization, Eqs. (7)-(8) ---

def test_group_maximum_lands_on_q_max_and_zero_group():
    r = _rng(3)
    x = r.standard_normal((5, 384)) * 3
    x[2, 128:256] = 0.0
    q, s = q8.quantize_activation(x)
    g = q.reshape(5, 3, 128)
    amax_idx = np.argmax(np.abs(x.reshape(5, 3, 128)), axis=2)
    for t in range(5):
        for j in range(3):
            if t == 2 and j == 1:
                assert s[t, j] == 0 and np.all(g[t, j] == 0)
            else:
                assert abs(g[t, j, amax_idx[t, j]]) == 448.0
                assert s[t, j] == np.float32(np.float32(np.abs(x[t, j * 128:(j + 1) * 128]).max()) / np.float32(448))


def test_power_of_two_scaling_and_group_independence():
    r = _rng(4)
    x = r.standard_normal((4, 256)).astype(np.float32).astype(np.float64)
    q, s = q8.quantize_activation(x)
    y = x.copy()
    y[:, :128] *= 2.0 ** 5                          # first group of every row, exact in fp32
    y[:, 128:] += 0.0
    q2, s2 = q8.quantize_activation(y)
    assert np.array_equal(q2, q) and np.array_equal(s2[:, 0], s[:, 0] * 32) and np.array_equal(s2[:, 1], s[:, 1])
    z = x.copy()
    z[:, 128:] = r.standard_normal((4, 128))       # another second group: the first is unchanged
    q3, s3 = q8.quantize_activation(z)
    assert np.array_equal(q3[:, :128], q[:, :128]) and np.array_equal(s3[:, 0], s[:, 0])


def test_quantization_error_within_the_format_bound():
    r = _rng(5)
    x = r.standard_normal((64, 512)) * np.exp2(r.integers(-4, 4, size=(64, 1)))
    q, s = q8.quantize_activation(x)
    deq = q8.dequantize_activation(q, s)
    sc = np.repeat(s, 128, axis=1)
    v = np.abs(x) / sc                               # position on the format's grid
    # normals: half a spacing is 2^-4 of the value's binade start; subnormals: 2^-10
    bound = np.where(v >= 2.0 ** -6, 2.0 ** -4 * v, 2.0 ** -10) * sc + 1e-7 * np.abs(x)
    assert np.all(np.abs(deq - x) <= bound)


def test_weight_blocks_are_independent_and_land_on_q_max():
    r = _rng(6)
    w = r.standard_normal((256, 384)) * 0.02
    q, s = q8.quantize_weight(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            blk = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert np.max(np.abs(blk)) == 448.0
    w2 = w.copy()
    w2[:128, :128] *= 7.0
    q2, s2 = q8.quantize_weight(w2)
    assert np.array_equal(q2[128:], q[128:]) and np.array_equal(q2[:128, 128:], q[:128, 128:])


# ------------------------------------------------------- the quantized linear ---

def test_fp8_linear_matches_torch_matmul_of_dequantized_operands():
    r = _rng(7)
    a = r.standard_normal((33, 256))
    w = r.standard_normal((384, 256)) * 0.05
    qa, sa = q8.quantize_activation(a)
    qw, sw = q8.quantize_weight(w)
    A = torch.from_numpy(qa) * torch.from_numpy(sa).repeat_interleave(128, dim=1)
    W = torch.from_numpy(qw) * torch.from_numpy(sw).repeat_interleave(128, 0).repeat_interleave(128, 1)
    np.testing.assert_allclose(q8.fp8_linear(qa, sa, qw, sw), (A @ W.T).numpy(), rtol=1e-13, atol=1e-13)


def test_fp8_linear_is_exact_on_grid_operands():
    # Operands already on the E4M3 grid times a power of two, with each group's
    # maximum at 448 * 2^j: quantization is exact and the product equals A W^T.
    r = _rng(8)
    vals = q8.e4m3_values()
    a = r.choice(vals, size=(16, 256)) * 2.0 ** -6
    w = r.choice(vals, size=(256, 256)) * 2.0 ** -10
    a[:, 0] = 448 * 2.0 ** -6
    a[:, 128] = -448 * 2.0 ** -6
    for i in range(2):
        for j in range(2):
            w[i * 128, j * 128] = 448 * 2.0 ** -10
    qa, sa = q8.quantize_activation(a)
    qw, sw = q8.quantize_weight(w)
    assert np.all(sa == 2.0 ** -6) and np.all(sw == 2.0 ** -10)
    np.testing.assert_array_equal(q8.fp8_linear(qa, sa, qw, sw), a @ w.T)


# ---------------------------------------------------------- AddNorm, SwiGLU ---

def test_add_norm_matches_torch_bf16_add_and_rms_norm():
    gen = torch.Generator().manual_seed(9)
    h = torch.randn(7, 256, generator=gen).to(torch.bfloat16)
    a = (0.3 * torch.randn(7, 256, generator=gen)).to(torch.bfloat16)
    g = (1 + 0.1 * torch.randn(256, generator=gen)).to(torch.bfloat16)
    rr, x = q8.add_norm(h.double().numpy(), a.double().numpy(), g.double().numpy(), 1e-5)
    np.testing.assert_array_equal(rr, (h + a).double().numpy())         # torch adds in fp32, rounds to bf16
    ref = F.rms_norm(torch.from_numpy(rr), (256,), g.double(), eps=1e-5).numpy()
    np.testing.assert_allclose(x, ref, rtol=1e-13, atol=1e-13)


def test_swiglu_matches_torch_silu():
    r = _rng(10)
    g, u = r.standard_normal((5, 64)) * 4, r.standard_normal((5, 64))
    ref = (F.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(q8.swiglu(g, u), ref, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ the FFN ---

def test_ffn_fp8_tracks_the_unquantized_ffn():
    # Per-group FP8 keeps every linear within a few percent: the FFN's down
    # projection agrees with the unquantized one to a small relative row error,
    # while swapping gate and up (a wiring mistake) does not.
    r = _rng(11)
    T, D, Fh = 24, 256, 384
    h = q8.round_bf16(r.standard_normal((T, D)))
    a = q8.round_bf16(0.5 * r.standard_normal((T, D)))
    g = q8.round_bf16(1 + 0.1 * r.standard_normal(D))
    wg, wu = [q8.round_bf16(0.05 * r.standard_normal((Fh, D))) for _ in range(2)]
    wd = q8.round_bf16(0.05 * r.standard_normal((D, Fh)))
    got = q8.ffn_fp8(h, a, g, wg, wu, wd, 1e-5)
    ref = q8.ffn_exact(h, a, g, wg, wu, wd, 1e-5)
    rel = np.linalg.norm(got["down"] - ref["down"], axis=1) / np.linalg.norm(ref["down"], axis=1)
    assert rel.max() < 0.12, rel.max()            # ~2^-4/sqrt(3) rms per quantized operand, two linears
    np.testing.assert_array_equal(got["r"], ref["r"])
    swapped = q8.ffn_exact(h, a, g, wu, wg, wd, 1e-5)
    rel_sw = np.linalg.norm(swapped["down"] - ref["down"], axis=1) / np.linalg.norm(ref["down"], axis=1)
    assert rel_sw.min() > 0.3
    # the output is the bf16 residual sum
    np.testing.assert_array_equal(got["out"], q8.round_bf16(got["r"] + got["down"]))
