"""CPU pins of the attention-only GPU check (tests/attn_check.py).

An emulation of the kernels' roundings (fp32 scores from fp16 operands, fp16
probabilities, fp32 accumulation, one final rounding of O to bf16) must pass
the check; the same emulation with one key dropped or counted twice at a tile
edge must fail it, at every length the workloads use.  No GPU is used.
"""

import numpy as np
import pytest
import torch

import attn_check


def _round_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _emulate(q, k, v, scale, keys):
    """fp32 softmax attention of rows q over the listed keys, probabilities rounded to fp16."""
    q32, k32, v32 = (np.asarray(x, np.float32) for x in (q, k[keys], v[keys]))
    s = (q32 @ k32.T) * np.float32(scale * np.log2(np.e))
    m = s.max(axis=1, keepdims=True)
    p = np.exp2(s - m).astype(np.float32)
    l = p.sum(axis=1, dtype=np.float32)
    o = p.astype(np.float16).astype(np.float32) @ v32
    out = _round_bf16(o / l[:, None])
    lse = ((m[:, 0] + np.log2(l)) * np.float32(np.log(2))).astype(np.float64)
    return out, lse


def _inputs(n, rows, d=128, seed=0):
    r = np.random.default_rng([20261202, 900, n, seed])
    # Magnitudes of the LLaDA-shaped workloads: q, k ~ 1.3, v ~ 1.3 per feature.
    q = (1.3 * r.standard_normal((rows, d))).astype(np.float16).astype(np.float64)
    k = (1.3 * r.standard_normal((n, d))).astype(np.float16).astype(np.float64)
    v = (1.3 * r.standard_normal((n, d))).astype(np.float16).astype(np.float64)
    return q, k, v


@pytest.mark.parametrize("n", [100, 768, 2304, 4864])
def test_emulated_kernel_passes_and_one_key_error_fails(n):
    rows, d = 64, 128
    scale = 1 / np.sqrt(d)
    q, k, v = _inputs(n, rows, d)
    o_ref, lse_ref, s_abs = attn_check.full_rows(q, k, v, scale)

    def check(keys):
        out, lse = _emulate(q, k, v, scale, keys)
        rep = attn_check.Report(p_bits=11)
        rep.add("emulated", out, o_ref, s_abs, n, 8, lse, lse_ref)
        return rep

    rep = check(np.arange(n))
    assert rep.worst_lse < 0.2 * attn_check.LSE_ATOL, rep.summary()
    edge = 64 if n > 64 else n // 2                      # first key of the second 64-key tile
    dropped = np.r_[0:edge, edge + 1:n]
    doubled = np.r_[0:n, edge]
    for keys, what in ((dropped, "dropped"), (doubled, "doubled")):
        with pytest.raises(AssertionError):
            check(keys)


def test_invariant_row_update_pins():
    # A step's invariant rows: FACache state over U keys (stored as fp16 O~/l
    # and fp32 m, l), updated with the block's keys; a block key lost from the
    # update fails the check, the faithful update passes.
    n, B, rows, d = 800, 32, 48, 128
    scale = 1 / np.sqrt(d)
    q, k, v = _inputs(n, rows, d, seed=1)
    U, C = np.arange(0, n - B), np.arange(n - B, n)
    import oracle
    m_c, l_c, O_c = oracle.state_over_keys(q, k[U], v[U], scale)
    o_c = (O_c / l_c[:, None]).astype(np.float16).astype(np.float64)
    o_ref, lse_ref, s_abs = attn_check.invariant_rows(q, m_c, l_c, o_c, k[C], v[C], scale)

    def emulate(cols):
        m, l, O = oracle.online_update((m_c, l_c, o_c * l_c[:, None]), q, k[cols], v[cols], scale)
        o, lse = oracle.finalize((m, l, O))
        return _round_bf16(o), lse

    rep = attn_check.Report()
    out, lse = emulate(C)
    rep.add("faithful", out, o_ref, s_abs, B, 8, lse, lse_ref)
    with pytest.raises(AssertionError):
        out, lse = emulate(C[1:])
        attn_check.Report().add("dropped", out, o_ref, s_abs, B, 8, lse, lse_ref)
