"""Plain CPU oracle of the rest of layer 0 and of the sampler cut.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

What it computes (LaCache, "Exact Caching and Precision-Adaptive Inference
for Diffusion Large Language Models", arXiv 2607.16339, Figure 2 and the
last paragraph of Section 3.4):

* The rest of layer 0 after its attention, in the parameter precision (the
  first layer is left out of the FP8 strategy, Section 3.4): the output
  projection W_o of the attention output, the residual add onto the layer's
  input rows (the EmbedCache rows H), the feed-forward RMSNorm, the gate-up
  linear, SwiGLU, the down (ffout) linear and the second residual add.  Every
  row of the sequence is computed: each row's attention output changes when
  the block's keys change.
* The sampler cut (Figure 2's caption; Section 3.4, last paragraph): only the
  current block's rows of the transformer output go through the final norm,
  the lm-head and the float softmax.  The cut is exact: every one of these
  operators acts on each row alone.

Readings where the pages are silent (each listed in the design doc):
* "Original precision" is a bf16 model: every operator's output is rounded
  to bf16 (round to nearest even), products and sums are exact before that
  rounding.  a = bf16(O W_o^T); r = bf16(h + a); x = bf16(gamma r / rms(r));
  gate = bf16(x W_g^T), up = bf16(x W_u^T); y = bf16(silu(gate) up);
  d = bf16(y W_d^T); out = bf16(r + d).  rms(r) = sqrt(mean(r^2) + eps), the
  form the attention's RMSNorm uses.
* The float softmax: logits = fp32(z W_lm^T) with z = bf16(gamma_f row /
  rms(row)) the final norm of a block row; probabilities softmax(logits); the
  sampler's token is the argmax (the lowest index among equal maxima) and its
  confidence the largest probability.
Everything else is fp64.
"""

from __future__ import annotations

import numpy as np

from .fp8_ref import round_bf16, silu

__all__ = [
    "linear", "rms_norm_rows", "o_proj_residual", "ffn_bf16", "layer0_finish", "block_rows", "final_norm",
    "lm_logits", "softmax_rows", "sample_rows", "sampler_cut", "sampler_all_rows",
]


def linear(x, w) -> np.ndarray:
    """x W^T in fp64 (x [T, K], w [N, K]): the exact product of bf16 values up to fp64 rounding."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def rms_norm_rows(r, gamma, eps: float) -> np.ndarray:
    """gamma * r / sqrt(mean(r^2) + eps), row by row, unrounded."""
    r = np.asarray(r, np.float64)
    return np.asarray(gamma, np.float64) * r / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)


def o_proj_residual(h, o, w_o):
    """a = bf16(O W_o^T), r = bf16(h + a).  h [T, D] (the layer's input rows),
    o [T, H d_h] (the attention output, heads concatenated), w_o [D, H d_h]."""
    a = round_bf16(linear(o, w_o))
    return a, round_bf16(np.asarray(h, np.float64) + a)


def ffn_bf16(r, gamma, w_gate, w_up, w_down, eps: float) -> dict:
    """The feed-forward half in bf16: x, gate, up, y, d, out = bf16(r + d)."""
    x = round_bf16(rms_norm_rows(r, gamma, eps))
    gate = round_bf16(linear(x, w_gate))
    up = round_bf16(linear(x, w_up))
    y = round_bf16(silu(gate) * up)
    d = round_bf16(linear(y, w_down))
    return dict(x=x, gate=gate, up=up, y=y, d=d, out=round_bf16(np.asarray(r, np.float64) + d))


def layer0_finish(h, o, w_o, gamma, w_gate, w_up, w_down, eps: float) -> dict:
    """Layer 0 after its attention, for every row: W_o, residual, FFN, residual."""
    a, r = o_proj_residual(h, o, w_o)
    f = ffn_bf16(r, gamma, w_gate, w_up, w_down, eps)
    f.update(a=a, r=r)
    return f


def block_rows(seqs) -> np.ndarray:
    """Flat row indices of the current blocks, sample by sample: seq_offset + [block_start, block_end)."""
    return np.concatenate([np.arange(s[0] + s[2], s[0] + s[3]) for s in seqs]).astype(np.int64)


def final_norm(rows, gamma_f, eps: float) -> np.ndarray:
    return round_bf16(rms_norm_rows(rows, gamma_f, eps))


def lm_logits(z, w_lm) -> np.ndarray:
    """fp32 logits of bf16 rows z against the lm-head w_lm [V, D] (exact product rounded once to fp32)."""
    return linear(z, w_lm).astype(np.float32).astype(np.float64)


def softmax_rows(logits) -> np.ndarray:
    l = np.asarray(logits, np.float64)
    e = np.exp(l - l.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sample_rows(hidden_rows, gamma_f, w_lm, eps: float) -> dict:
    """Final norm, lm-head and float softmax of the given rows; the argmax token and its probability."""
    z = final_norm(hidden_rows, gamma_f, eps)
    logits = lm_logits(z, w_lm)
    p = softmax_rows(logits)
    token = np.argmax(logits, axis=-1)                 # first index among equal maxima
    return dict(z=z, logits=logits, probs=p, token=token, confidence=p[np.arange(len(p)), token])


def sampler_cut(hidden, seqs, gamma_f, w_lm, eps: float) -> dict:
    """The sampler on the current blocks' rows only (the cut)."""
    rows = block_rows(seqs)
    out = sample_rows(np.asarray(hidden, np.float64)[rows], gamma_f, w_lm, eps)
    out["rows"] = rows
    return out


def sampler_all_rows(hidden, gamma_f, w_lm, eps: float) -> dict:
    """The sampler without the cut: every row of the transformer output."""
    return sample_rows(hidden, gamma_f, w_lm, eps)
