"""Seeded synthetic inputs for the layer-0 cached block step.

This module only draws inputs: model parameters, token ids, the per-sample
block table and the per-step edits of the current block.  It holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle may take their
inputs from it.

Shapes follow the workloads of the pages: a LLaDA-8B-shaped first layer
(d_model 4096, 32 heads of 128, vocabulary 126464) decoded semi-autoregressively
in blocks of 32 or 64 (LaCache Appendix B.1; the DualCache layout
``[prompt | block 0 | ... | block K-1]``), plus a tiny fp32 model.  No dataset
content is used: token ids are uniform, parameters are Gaussian.

Seeding: every array comes from ``numpy.random.default_rng([BASE_SEED, a, b,
...])`` with a fixed stream tuple, so any row block of the embedding table can
be regenerated on its own.  Parameters are drawn in float32 and, for bf16
workloads, rounded to bf16 (round-to-nearest-even) here, so both sides see
exactly the same values.
"""

from __future__ import annotations

import functools
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

BASE_SEED = 20261202
_EMBED_CHUNK = 4096           # embedding rows per generator stream

# stream ids inside a parameter family / workload
_S_EMBED, _S_W, _S_GAMMA, _S_IDS, _S_LAYOUT, _S_EDIT = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    """One decoding configuration: model shape, batch layout and edit rule."""

    name: str
    dtype: str                      # "f32" or "bf16": storage dtype of params/caches
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    rope_theta: float
    batch: int
    prompt_lens: tuple              # per sample
    gen_len: int
    block_size: int
    block_idx: tuple                # per sample: index of the current block
    steps: int                      # inner denoising steps after the refresh
    edits: tuple                    # (lo, hi): ids changed per step, inclusive
    embed_std: float
    w_std: float = 0.02
    gamma_std: float = 0.1
    rms_eps: float = 1e-5
    param_family: int = 0           # parameters are shared by workloads of one family
    seed: int = 0                   # stream id of the ids / edits

    @property
    def seq_lens(self):
        return tuple(p + self.gen_len for p in self.prompt_lens)

    @property
    def n_features(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def total_tokens(self):
        return sum(self.seq_lens)

    @property
    def block_tokens(self):
        return self.batch * self.block_size

    def table(self):
        """Block table rows (seq_offset, seq_len, block_start, block_end)."""
        rows, off = [], 0
        for p, n, k in zip(self.prompt_lens, self.seq_lens, self.block_idx):
            bs = p + k * self.block_size
            rows.append((off, n, bs, bs + self.block_size))
            off += n
        return rows


def _draw_layout(name, batch, prompt_fn, nblocks, stream):
    rng = np.random.default_rng([BASE_SEED, stream, _S_LAYOUT])
    prompts = prompt_fn(rng)
    idx = tuple(int(x) for x in rng.integers(0, nblocks, size=batch))
    return tuple(int(p) for p in prompts), idx


def _make_workloads():
    llada = dict(d_model=4096, n_heads=32, n_kv_heads=32, head_dim=128, vocab=126464,
                 rope_theta=500000.0, embed_std=1.0, param_family=2, dtype="bf16")
    tiny = dict(d_model=256, n_heads=4, n_kv_heads=4, head_dim=64, vocab=512,
                rope_theta=10000.0, embed_std=0.02, param_family=1, dtype="f32")
    w = {}
    # Tiny fp32 cached step: prompt 64 + gen 64 in 4 blocks of 16, block 1,
    # 3 inner steps each re-drawing 4 ids.
    w["tiny"] = Workload(name="tiny", batch=1, prompt_lens=(64,), gen_len=64, block_size=16,
                         block_idx=(1,), steps=3, edits=(4, 4), seed=1, **tiny)
    # LLaDA-8B-shaped layer 0, batch 1: prompt 512 + gen 256, blocks of 32, block 3.
    w["llada8b"] = Workload(name="llada8b", batch=1, prompt_lens=(512,), gen_len=256,
                            block_size=32, block_idx=(3,), steps=20, edits=(2, 8), seed=2, **llada)
    # Batch 16, prompt 256 + gen 256, blocks of 32, current block uniform in 0..7.
    _, idx16 = _draw_layout("batched16", 16, lambda r: [256] * 16, 8, 3)
    w["batched16"] = Workload(name="batched16", batch=16, prompt_lens=(256,) * 16, gen_len=256,
                              block_size=32, block_idx=idx16, steps=20, edits=(2, 8), seed=3, **llada)
    w["tiny_batched16"] = Workload(name="tiny_batched16", batch=16, prompt_lens=(256,) * 16,
                                   gen_len=256, block_size=32, block_idx=idx16, steps=3,
                                   edits=(2, 8), seed=6, **tiny)
    # Long context: batch 4, prompt 3840 + gen 1024, blocks of 64, block 8.
    w["long4"] = Workload(name="long4", batch=4, prompt_lens=(3840,) * 4, gen_len=1024,
                          block_size=64, block_idx=(8,) * 4, steps=20, edits=(2, 8), seed=4, **llada)
    # Variable-length batch: 32 samples, prompts uniform in [128, 2048], gen 256, blocks of 32.
    p32, idx32 = _draw_layout("varlen32", 32, lambda r: r.integers(128, 2049, size=32), 8, 5)
    w["varlen32"] = Workload(name="varlen32", batch=32, prompt_lens=p32, gen_len=256,
                             block_size=32, block_idx=idx32, steps=20, edits=(2, 8), seed=5, **llada)
    return w


WORKLOADS = _make_workloads()
# The five configurations in the order they are usually quoted.
CONFIG_ORDER = ("tiny", "llada8b", "batched16", "long4", "varlen32")


def custom(name, *, dtype="bf16", d_model=512, n_heads=4, n_kv_heads=None, head_dim=128,
           vocab=1000, rope_theta=10000.0, prompt_lens=(40,), gen_len=64, block_size=16,
           block_idx=None, steps=2, edits=(1, 4), embed_std=1.0, seed=100, param_family=None):
    """A small workload with arbitrary shapes (tests: ragged tails, several tiles)."""
    batch = len(prompt_lens)
    nblocks = -(-gen_len // block_size)
    if block_idx is None:
        rng = np.random.default_rng([BASE_SEED, seed, _S_LAYOUT])
        block_idx = tuple(int(x) for x in rng.integers(0, nblocks, size=batch))
    fam = param_family if param_family is not None else 1000 + seed
    return Workload(name=name, dtype=dtype, d_model=d_model, n_heads=n_heads,
                    n_kv_heads=n_kv_heads or n_heads, head_dim=head_dim, vocab=vocab,
                    rope_theta=rope_theta, batch=batch, prompt_lens=tuple(prompt_lens),
                    gen_len=gen_len, block_size=block_size, block_idx=tuple(block_idx),
                    steps=steps, edits=edits, embed_std=embed_std, param_family=fam, seed=seed)


# ----------------------------------------------------------------------------
# Rounding of drawn values to the storage dtype
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly representable in bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


def _store(x, dtype):
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


# ----------------------------------------------------------------------------
# Parameters
# ----------------------------------------------------------------------------

def _param_key(wl: Workload):
    return (wl.param_family, wl.dtype, wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim,
            wl.vocab, wl.embed_std, wl.w_std, wl.gamma_std)


@functools.lru_cache(maxsize=4)
def _params_cached(key):
    fam, dtype, D, H, Hk, d, V, e_std, w_std, g_std = key
    F = (H + 2 * Hk) * d
    E = np.empty((V, D), np.float32)

    def fill(c):
        r0, r1 = c * _EMBED_CHUNK, min(V, (c + 1) * _EMBED_CHUNK)
        rng = np.random.default_rng([BASE_SEED, fam, _S_EMBED, c])
        E[r0:r1] = _store(rng.standard_normal((r1 - r0, D), dtype=np.float32) * np.float32(e_std), dtype)

    nchunks = -(-V // _EMBED_CHUNK)
    with ThreadPoolExecutor(max_workers=min(16, nchunks)) as ex:
        list(ex.map(fill, range(nchunks)))
    rng = np.random.default_rng([BASE_SEED, fam, _S_W])
    W = _store(rng.standard_normal((F, D), dtype=np.float32) * np.float32(w_std), dtype)
    rng = np.random.default_rng([BASE_SEED, fam, _S_GAMMA])
    gamma = _store(1.0 + rng.standard_normal(D, dtype=np.float32) * np.float32(g_std), dtype)
    for a in (E, W, gamma):
        a.setflags(write=False)
    return {"embed": E, "gamma": gamma, "w_qkv": W}


def params(wl: Workload) -> dict:
    """Embedding table E [V, D], RMSNorm gain gamma [D], W_qkv [F, D] (float32 arrays).

    W_qkv rows: Q heads, then K heads, then V heads, d_h rows per head.
    Values are exactly representable in the workload dtype.
    """
    return _params_cached(_param_key(wl))


# ----------------------------------------------------------------------------
# Token ids and the edit schedule
# ----------------------------------------------------------------------------

def initial_ids(wl: Workload) -> np.ndarray:
    """Flat token ids [T]: each sample's [prompt | blocks], uniform over the vocabulary."""
    rng = np.random.default_rng([BASE_SEED, 100 + wl.seed, _S_IDS])
    return rng.integers(0, wl.vocab, size=wl.total_tokens, dtype=np.int64).astype(np.int32)


def step_ids(wl: Workload, ids_prev: np.ndarray, step: int):
    """Ids after inner step ``step`` (1-based): in every sample's current block,
    k ~ U{lo..hi} distinct positions get fresh uniform ids.

    Returns (ids [T], block_ids [sum B_b]) with block ids concatenated in sample order.
    """
    rng = np.random.default_rng([BASE_SEED, 100 + wl.seed, _S_EDIT, step])
    ids = np.array(ids_prev, dtype=np.int32, copy=True)
    blocks = []
    for (off, n, bs, be) in wl.table():
        B = be - bs
        k = int(rng.integers(wl.edits[0], wl.edits[1] + 1))
        pos = rng.choice(B, size=min(k, B), replace=False)
        ids[off + bs + pos] = rng.integers(0, wl.vocab, size=len(pos))
        blocks.append(ids[off + bs: off + be])
    return ids, np.concatenate(blocks).astype(np.int32)


def block_ids_of(wl: Workload, ids: np.ndarray) -> np.ndarray:
    """The current blocks' ids [sum B_b] cut out of flat ids [T]."""
    return np.concatenate([ids[off + bs: off + be] for (off, n, bs, be) in wl.table()]).astype(np.int32)


def with_steps(wl: Workload, steps: int) -> Workload:
    return replace(wl, steps=steps)


# ----------------------------------------------------------------------------
# The FFN of a layer after the first (per-group FP8): weights and inputs
# ----------------------------------------------------------------------------

# LLaDA-8B's feed-forward width (SwiGLU, d_model 4096).
LLADA_D_FF = 12288
_S_FFN_W, _S_FFN_X = 6, 7
_S_LAYER_W, _S_LM = 8, 9
# LLaDA-8B's vocabulary (the lm-head rows).
LLADA_VOCAB = 126464


def ffn_params(d_model: int, d_ff: int, family: int = 0) -> dict:
    """RMSNorm gain gamma [D] ~ 1 + N(0, 0.1), w_gate, w_up [F, D] and w_down
    [D, F] ~ N(0, 0.02), drawn in fp32 and rounded to bf16 (float32 arrays)."""
    rng = np.random.default_rng([BASE_SEED, 50 + family, _S_FFN_W, d_model, d_ff])
    gamma = round_to_bf16(1.0 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1))
    w_gate = round_to_bf16(rng.standard_normal((d_ff, d_model), dtype=np.float32) * np.float32(0.02))
    w_up = round_to_bf16(rng.standard_normal((d_ff, d_model), dtype=np.float32) * np.float32(0.02))
    w_down = round_to_bf16(rng.standard_normal((d_model, d_ff), dtype=np.float32) * np.float32(0.02))
    return {"gamma": gamma, "w_gate": w_gate, "w_up": w_up, "w_down": w_down}


def ffn_inputs(n_rows: int, d_model: int, seed: int = 0):
    """The residual stream h [T, D] ~ N(0, 1) and the attention block's output
    a [T, D] ~ N(0, 0.5^2), bf16 values (float32 arrays)."""
    rng = np.random.default_rng([BASE_SEED, 60 + seed, _S_FFN_X, n_rows, d_model])
    h = round_to_bf16(rng.standard_normal((n_rows, d_model), dtype=np.float32))
    a = round_to_bf16(rng.standard_normal((n_rows, d_model), dtype=np.float32) * np.float32(0.5))
    return h, a


def layer_params(d_model: int, hd: int, d_ff: int, family: int = 0) -> dict:
    """The rest of a layer: w_o [D, hd] ~ N(0, 0.02) and the FFN of ffn_params
    (gamma, w_gate, w_up, w_down), bf16 values (float32 arrays)."""
    rng = np.random.default_rng([BASE_SEED, 70 + family, _S_LAYER_W, d_model, hd])
    w_o = round_to_bf16(rng.standard_normal((d_model, hd), dtype=np.float32) * np.float32(0.02))
    p = ffn_params(d_model, d_ff, 100 + family)
    p["w_o"] = w_o
    return p


def lm_head_params(d_model: int, vocab: int, family: int = 0) -> dict:
    """Final norm gain gamma_f [D] ~ 1 + N(0, 0.1) and the lm-head w_lm
    [vocab, D] ~ N(0, 0.02), drawn 8192 rows per generator stream (so rows can
    be regenerated alone), bf16 values (float32 arrays)."""
    rng = np.random.default_rng([BASE_SEED, 80 + family, _S_LM, d_model, vocab])
    gamma_f = round_to_bf16(1.0 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1))
    w = np.empty((vocab, d_model), np.float32)
    for r0 in range(0, vocab, 8192):
        g = np.random.default_rng([BASE_SEED, 80 + family, _S_LM, d_model, vocab, r0])
        n = min(8192, vocab - r0)
        w[r0:r0 + n] = g.standard_normal((n, d_model), dtype=np.float32) * np.float32(0.02)
    return {"gamma_f": gamma_f, "w_lm": round_to_bf16(w)}


def multilayer_params(d_model: int, n_heads: int, head_dim: int, d_ff: int, n_layers: int, vocab: int,
                      qkv_std: float = 0.02, family: int = 0) -> dict:
    """A model of n_layers layers of one shape (bf16 values, float32 arrays):
    the embedding E [vocab, D] ~ N(0, 1); per layer the attention RMSNorm gain
    ~ 1 + N(0, 0.1), W_qkv [3 H d_h, D] ~ N(0, qkv_std^2) (rows: Q heads, K
    heads, V heads), and the rest of the layer as layer_params."""
    rng = np.random.default_rng([BASE_SEED, 90 + family, d_model, n_heads, n_layers, vocab])
    p = {"embed": round_to_bf16(rng.standard_normal((vocab, d_model), dtype=np.float32)), "layers": []}
    for li in range(n_layers):
        r = np.random.default_rng([BASE_SEED, 90 + family, d_model, n_heads, n_layers, vocab, li])
        lp = layer_params(d_model, n_heads * head_dim, d_ff, 1000 * (family + 1) + li)
        lp["gamma_ffn"] = lp.pop("gamma")
        lp["gamma_attn"] = round_to_bf16(1.0 + r.standard_normal(d_model, dtype=np.float32) * np.float32(0.1))
        lp["w_qkv"] = round_to_bf16(r.standard_normal((3 * n_heads * head_dim, d_model), dtype=np.float32)
                                    * np.float32(qkv_std))
        p["layers"].append(lp)
    return p
