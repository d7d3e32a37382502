"""Thin Python binding of liblacache.so (include/lacache.h).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and contiguity and handed to the C ABI as raw pointers together with
the current HIP stream.  Every step of the computation runs in the HIP
kernels; there is no Python or CPU fallback, and a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblacache.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
OP_PREFILL, OP_BLOCK_STEP, OP_DUALCACHE_ATTN, OP_REFRESH_BLOCK, OP_PROJECT_BLOCK = 0, 1, 2, 3, 4
DEVFLAG_BAD_TOKEN_ID = 1
DEVFLAG_CACHE_RANGE = 2
DEVFLAG_SEARCH_ORDER = 4

EXPORTED = ("lacache_create", "lacache_destroy", "lacache_workspace_size", "lacache_prefill_cache",
            "lacache_block_step", "lacache_refresh_block", "lacache_dualcache_attn", "lacache_read_device_status",
            "lacache_profile_enable", "lacache_profile_read", "lacache_status_string", "lacache_last_error",
            "lacache_packed_weight_size", "lacache_pack_qkv_weight", "lacache_block_step_noalloc",
            "lacache_ffn_weight_bytes", "lacache_ffn_pack_weights", "lacache_ffn_workspace_size", "lacache_ffn_fp8",
            "lacache_layer_finish_workspace_size", "lacache_layer_finish", "lacache_sampler_workspace_size",
            "lacache_sampler_cut", "lacache_project_block", "lacache_track_workspace_size",
            "lacache_track_select", "lacache_verify_attn", "lacache_verify_accept")
(KERNEL_QKV, KERNEL_BLOCK_ROWS, KERNEL_INVARIANT_ROWS, KERNEL_MERGE, KERNEL_REFRESH_ATTN, KERNEL_QKV_PREP,
 KERNEL_QKV_GEMM, KERNEL_ATTN, KERNEL_FFN_NORM, KERNEL_FFN_GATE_UP, KERNEL_FFN_DOWN, KERNEL_LAYER_OPROJ,
 KERNEL_LAYER_NORM, KERNEL_LAYER_GATE_UP, KERNEL_LAYER_DOWN, KERNEL_SAMPLER_NORM, KERNEL_SAMPLER_LMHEAD,
 KERNEL_SAMPLER_SOFTMAX, KERNEL_TRACK_IMPORTANCE, KERNEL_TRACK_SELECT, KERNEL_VERIFY_ATTN,
 KERNEL_VERIFY_ACCEPT) = range(22)
KERNEL_NAMES = ("qkv", "block_rows", "invariant_rows", "merge", "refresh_attn", "qkv_prep", "qkv_gemm", "attn",
                "ffn_norm", "ffn_gate_up", "ffn_down", "layer_oproj", "layer_norm", "layer_gate_up", "layer_down",
                "sampler_norm", "sampler_lmhead", "sampler_softmax", "track_importance", "track_select",
                "verify_attn", "verify_accept")


class Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("w_qkv_packed", ctypes.c_void_p)]


class Cache(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("l", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("n_rows", ctypes.c_int64)]


class FfnWeights(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_void_p), ("gate_up", ctypes.c_void_p), ("s_gate_up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_o", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class Seq(ctypes.Structure):
    _fields_ = [("seq_offset", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("block_start", ctypes.c_int32), ("block_end", ctypes.c_int32)]


class LaCacheError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblacache.so and declare its signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_state_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "lacache_create": (st, [ctypes.POINTER(Config), ctypes.POINTER(P)]),
        "lacache_destroy": (st, [P]),
        "lacache_workspace_size": (st, [P, I32, ctypes.POINTER(Seq), I32, ctypes.POINTER(SZ)]),
        "lacache_prefill_cache": (st, [P, ctypes.POINTER(Weights), P, ctypes.POINTER(Seq), I32,
                                       ctypes.POINTER(Cache), P, P, P, SZ, P]),
        "lacache_block_step": (st, [P, ctypes.POINTER(Weights), P, ctypes.POINTER(Seq), I32,
                                    ctypes.POINTER(Cache), P, P, P, SZ, P]),
        "lacache_block_step_noalloc": (st, [P, ctypes.POINTER(Weights), P, ctypes.POINTER(Seq), I32,
                                            ctypes.POINTER(Cache), P, P, P]),
        "lacache_refresh_block": (st, [P, ctypes.POINTER(Weights), P, ctypes.POINTER(Seq), ctypes.POINTER(Seq), I32,
                                       ctypes.POINTER(Cache), P, P, P, SZ, P]),
        "lacache_dualcache_attn": (st, [P, P, P, P, I64, ctypes.POINTER(Seq), I32, P, P, P, SZ, P]),
        "lacache_packed_weight_size": (st, [P, ctypes.POINTER(SZ)]),
        "lacache_pack_qkv_weight": (st, [P, P, P, SZ, P]),
        "lacache_ffn_weight_bytes": (st, [P, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ),
                                          ctypes.POINTER(SZ)]),
        "lacache_ffn_pack_weights": (st, [P, I32, P, P, P, P, P, P, P, P]),
        "lacache_ffn_workspace_size": (st, [P, I32, I64, I32, ctypes.POINTER(SZ)]),
        "lacache_ffn_fp8": (st, [P, I32, ctypes.POINTER(FfnWeights), P, P, I64, P, P, P, SZ, P]),
        "lacache_project_block": (st, [P, ctypes.POINTER(Weights), P, ctypes.POINTER(Seq), I32,
                                       ctypes.POINTER(Cache), P, SZ, P]),
        "lacache_track_workspace_size": (st, [P, I64, ctypes.POINTER(SZ)]),
        "lacache_track_select": (st, [P, ctypes.POINTER(Cache), P, ctypes.POINTER(Seq), I32, I32, P, P, P, SZ, P]),
        "lacache_verify_attn": (st, [P, P, P, P, P, P, ctypes.POINTER(I32), ctypes.POINTER(Cache), ctypes.POINTER(Seq),
                                     I32, P, P, P]),
        "lacache_verify_accept": (st, [P, P, P, P, P, ctypes.POINTER(I32), ctypes.POINTER(Seq), I32, ctypes.c_float,
                                       P, P, P]),
        "lacache_layer_finish_workspace_size": (st, [P, I32, I64, I32, ctypes.POINTER(SZ)]),
        "lacache_layer_finish": (st, [P, I32, ctypes.POINTER(LayerWeights), P, P, I64, P, P, P, SZ, P]),
        "lacache_sampler_workspace_size": (st, [P, I32, ctypes.POINTER(Seq), I32, ctypes.POINTER(SZ)]),
        "lacache_sampler_cut": (st, [P, P, I64, ctypes.POINTER(Seq), I32, P, P, I32, P, P, P, P, SZ, P]),
        "lacache_read_device_status": (st, [P, P, ctypes.POINTER(ctypes.c_uint32)]),
        "lacache_profile_enable": (st, [P, ctypes.c_int]),
        "lacache_profile_read": (st, [P, I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
        "lacache_status_string": (ctypes.c_char_p, [st]),
        "lacache_last_error": (ctypes.c_char_p, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _seqs(table):
    arr = (Seq * len(table))()
    for i, (off, n, bs, be) in enumerate(table):
        arr[i] = Seq(int(off), int(n), int(bs), int(be))
    return arr


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}
# RoPECache element type: fp32 for fp32 parameters, fp16 for bf16 parameters.
_CACHE_DTYPE = {F32: torch.float32, BF16: torch.float16}


@dataclass
class CacheTensors:
    """Caller-owned device buffers of the caches, the output and the LSE."""

    h: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    m: torch.Tensor
    l: torch.Tensor
    o: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor

    @property
    def n_rows(self):
        return self.h.shape[0]


class Context:
    """One lacache_ctx: layer-0 shape, RoPE table, device status word."""

    def __init__(self, d_model, n_heads, n_kv_heads, head_dim, vocab, max_seq_len, rope_theta,
                 rms_eps=1e-5, sm_scale=0.0, dtype="bf16"):
        self.lib = load_library()
        self.dtype_code = BF16 if dtype in ("bf16", BF16, torch.bfloat16) else F32
        self.torch_dtype = _TORCH_DTYPE[self.dtype_code]
        self.cache_dtype = _CACHE_DTYPE[self.dtype_code]
        self.cfg = Config(d_model, n_heads, n_kv_heads, head_dim, vocab, max_seq_len, rope_theta, rms_eps,
                          sm_scale, self.dtype_code)
        h = ctypes.c_void_p()
        st = self.lib.lacache_create(ctypes.byref(self.cfg), ctypes.byref(h))
        if st != OK:
            raise LaCacheError(st, "lacache_create: " + self.lib.lacache_status_string(st).decode())
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.lacache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------
    def _check(self, st, what):
        if st != OK:
            msg = self.lib.lacache_last_error(self.handle).decode()
            raise LaCacheError(st, f"{what}: {msg}")

    def alloc_cache(self, n_rows, device="cuda"):
        """Allocate (uninitialised) cache, output and LSE buffers of n_rows rows."""
        c = self.cfg
        dt, ct = self.torch_dtype, self.cache_dtype
        e = dict(device=device)
        return CacheTensors(
            h=torch.empty(n_rows, c.d_model, dtype=dt, **e),
            q=torch.empty(n_rows, c.n_heads, c.head_dim, dtype=ct, **e),
            k=torch.empty(n_rows, c.n_kv_heads, c.head_dim, dtype=ct, **e),
            v=torch.empty(n_rows, c.n_kv_heads, c.head_dim, dtype=ct, **e),
            m=torch.empty(n_rows, c.n_heads, dtype=torch.float32, **e),
            l=torch.empty(n_rows, c.n_heads, dtype=torch.float32, **e),
            o=torch.empty(n_rows, c.n_heads, c.head_dim, dtype=ct, **e),
            out=torch.empty(n_rows, c.n_heads, c.head_dim, dtype=dt, **e),
            lse=torch.empty(n_rows, c.n_heads, dtype=torch.float32, **e),
        )

    def workspace_size(self, op, table):
        n = ctypes.c_size_t()
        seqs = _seqs(table)
        self._check(self.lib.lacache_workspace_size(self.handle, op, seqs, len(table), ctypes.byref(n)),
                    "lacache_workspace_size")
        return n.value

    def alloc_workspace(self, op, table, device="cuda"):
        n = self.workspace_size(op, table)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def _weights(self, embed, gamma, w_qkv, w_qkv_packed=None):
        for name, t in (("embed", embed), ("gamma", gamma), ("w_qkv", w_qkv)):
            if t.dtype != self.torch_dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {self.torch_dtype} CUDA tensor")
        if w_qkv_packed is not None and (not w_qkv_packed.is_cuda or not w_qkv_packed.is_contiguous()):
            raise ValueError("w_qkv_packed must be a contiguous CUDA tensor")
        return Weights(embed.data_ptr(), gamma.data_ptr(), w_qkv.data_ptr(),
                       None if w_qkv_packed is None else w_qkv_packed.data_ptr())

    def packed_weight_size(self):
        """Bytes of the packed projection weight (0: this configuration has none)."""
        n = ctypes.c_size_t()
        self._check(self.lib.lacache_packed_weight_size(self.handle, ctypes.byref(n)), "lacache_packed_weight_size")
        return n.value

    def pack_qkv_weight(self, w_qkv, stream=None):
        """fp16 copy of w_qkv in the projection's tile order (uint8 CUDA tensor), or None if unsupported."""
        n = self.packed_weight_size()
        if n == 0:
            return None
        if w_qkv.dtype != self.torch_dtype or not w_qkv.is_cuda or not w_qkv.is_contiguous():
            raise ValueError(f"w_qkv must be a contiguous {self.torch_dtype} CUDA tensor")
        out = torch.empty(n, dtype=torch.uint8, device=w_qkv.device)
        self._check(self.lib.lacache_pack_qkv_weight(self.handle, _ptr(w_qkv), _ptr(out), n, _stream(stream)),
                    "lacache_pack_qkv_weight")
        return out

    @staticmethod
    def _cache(ct: CacheTensors):
        return Cache(ct.h.data_ptr(), ct.q.data_ptr(), ct.k.data_ptr(), ct.v.data_ptr(), ct.m.data_ptr(),
                     ct.l.data_ptr(), ct.o.data_ptr(), ct.n_rows)

    @staticmethod
    def _ids(t):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("token ids must be a contiguous int32 CUDA tensor")
        return t

    def prefill_cache(self, weights, ids, table, ct: CacheTensors, workspace=None, stream=None, lse=True):
        w = self._weights(*weights)
        seqs = _seqs(table)
        cache = self._cache(ct)
        ws = workspace
        st = self.lib.lacache_prefill_cache(self.handle, ctypes.byref(w), _ptr(self._ids(ids)), seqs, len(table),
                                            ctypes.byref(cache), _ptr(ct.out), _ptr(ct.lse) if lse else None,
                                            _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
        self._check(st, "lacache_prefill_cache")

    def block_step(self, weights, block_ids, table, ct: CacheTensors, workspace, stream=None, lse=True):
        w = self._weights(*weights)
        seqs = _seqs(table)
        cache = self._cache(ct)
        st = self.lib.lacache_block_step(self.handle, ctypes.byref(w), _ptr(self._ids(block_ids)), seqs,
                                         len(table), ctypes.byref(cache), _ptr(ct.out),
                                         _ptr(ct.lse) if lse else None, _ptr(workspace),
                                         0 if workspace is None else workspace.numel(), _stream(stream))
        self._check(st, "lacache_block_step")

    def project_block(self, weights, block_ids, table, ct: CacheTensors, workspace=None, stream=None):
        """lacache_project_block: a1-a5 for the block rows (RoPECache q, k, v and EmbedCache), no attention."""
        w = self._weights(*weights)
        seqs = _seqs(table)
        cache = self._cache(ct)
        st = self.lib.lacache_project_block(self.handle, ctypes.byref(w), _ptr(self._ids(block_ids)), seqs, len(table),
                                            ctypes.byref(cache), _ptr(workspace),
                                            0 if workspace is None else workspace.numel(), _stream(stream))
        self._check(st, "lacache_project_block")

    def block_step_noalloc(self, weights, block_ids, table, ct: CacheTensors, stream=None, lse=True):
        """lacache_block_step_noalloc: the block step on the library's static scratch (no workspace)."""
        w = self._weights(*weights)
        seqs = _seqs(table)
        cache = self._cache(ct)
        st = self.lib.lacache_block_step_noalloc(self.handle, ctypes.byref(w), _ptr(self._ids(block_ids)), seqs,
                                                 len(table), ctypes.byref(cache), _ptr(ct.out),
                                                 _ptr(ct.lse) if lse else None, _stream(stream))
        self._check(st, "lacache_block_step_noalloc")

    def refresh_block(self, weights, proj_ids, proj_table, table, ct: CacheTensors, workspace=None, stream=None,
                      lse=True):
        """Block-boundary refresh: re-project the rows of proj_table's blocks (ids proj_ids), then the full
        refresh attention for the block table `table`."""
        if len(proj_table) != len(table):
            raise ValueError("proj_table and table must have one row per sample each")
        w = self._weights(*weights)
        cache = self._cache(ct)
        st = self.lib.lacache_refresh_block(self.handle, ctypes.byref(w), _ptr(self._ids(proj_ids)), _seqs(proj_table),
                                            _seqs(table), len(table), ctypes.byref(cache), _ptr(ct.out),
                                            _ptr(ct.lse) if lse else None, _ptr(workspace),
                                            0 if workspace is None else workspace.numel(), _stream(stream))
        self._check(st, "lacache_refresh_block")

    def dualcache_attn(self, q_block, k, v, table, out_block, lse_block=None, workspace=None, stream=None):
        for name, t, dt in (("q_block", q_block, self.cache_dtype), ("k", k, self.cache_dtype),
                            ("v", v, self.cache_dtype), ("out_block", out_block, self.torch_dtype)):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor")
        seqs = _seqs(table)
        st = self.lib.lacache_dualcache_attn(self.handle, _ptr(q_block), _ptr(k), _ptr(v), k.shape[0], seqs,
                                             len(table), _ptr(out_block), _ptr(lse_block), _ptr(workspace),
                                             0 if workspace is None else workspace.numel(), _stream(stream))
        self._check(st, "lacache_dualcache_attn")

    # ------------------------------------------------------------------
    # Per-group FP8 FFN of the layers after the first
    def ffn_pack_weights(self, d_ff, w_gate, w_up, w_down, stream=None):
        """Quantize a layer's FFN weights (bf16 CUDA tensors) to the packed FP8 form:
        returns (gate_up uint8, s_gate_up float32, down uint8, s_down float32) CUDA tensors."""
        n = [ctypes.c_size_t() for _ in range(4)]
        self._check(self.lib.lacache_ffn_weight_bytes(self.handle, d_ff, *[ctypes.byref(x) for x in n]),
                    "lacache_ffn_weight_bytes")
        D = self.cfg.d_model
        for name, t, shape in (("w_gate", w_gate, (d_ff, D)), ("w_up", w_up, (d_ff, D)), ("w_down", w_down, (D, d_ff))):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor of shape {shape}")
        dev = w_gate.device
        gu = torch.empty(n[0].value, dtype=torch.uint8, device=dev)
        sgu = torch.empty(n[1].value // 4, dtype=torch.float32, device=dev)
        dn = torch.empty(n[2].value, dtype=torch.uint8, device=dev)
        sdn = torch.empty(n[3].value // 4, dtype=torch.float32, device=dev)
        self._check(self.lib.lacache_ffn_pack_weights(self.handle, d_ff, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                      _ptr(gu), _ptr(sgu), _ptr(dn), _ptr(sdn), _stream(stream)),
                    "lacache_ffn_pack_weights")
        return gu, sgu, dn, sdn

    def ffn_workspace(self, d_ff, n_rows, keeps_residual=True, device="cuda"):
        n = ctypes.c_size_t()
        self._check(self.lib.lacache_ffn_workspace_size(self.handle, d_ff, n_rows, int(bool(keeps_residual)),
                                                        ctypes.byref(n)), "lacache_ffn_workspace_size")
        return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)

    def ffn_fp8(self, d_ff, gamma, packed, h, attn_out, out, r_out=None, workspace=None, stream=None):
        """One FP8 FFN sub-block: out = bf16(r + down(swiglu(gate_up(RMSNorm(r))))) with r = bf16(h + attn_out)."""
        gu, sgu, dn, sdn = packed
        for name, t in (("gamma", gamma), ("h", h), ("attn_out", attn_out), ("out", out)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
        if h.shape != attn_out.shape or h.shape != out.shape or (r_out is not None and r_out.shape != h.shape):
            raise ValueError("h, attn_out, out (and r_out) must have the same shape [n_rows, d_model]")
        w = FfnWeights(gamma.data_ptr(), gu.data_ptr(), sgu.data_ptr(), dn.data_ptr(), sdn.data_ptr())
        ws = workspace if workspace is not None else self.ffn_workspace(d_ff, h.shape[0], r_out is not None, h.device)
        st = self.lib.lacache_ffn_fp8(self.handle, d_ff, ctypes.byref(w), _ptr(h), _ptr(attn_out), h.shape[0],
                                      _ptr(r_out), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
        self._check(st, "lacache_ffn_fp8")
        return ws

    def layer_workspace(self, d_ff, n_rows, keeps_residual=True, device="cuda"):
        n = ctypes.c_size_t()
        self._check(self.lib.lacache_layer_finish_workspace_size(self.handle, d_ff, n_rows, int(bool(keeps_residual)),
                                                                 ctypes.byref(n)), "lacache_layer_finish_workspace_size")
        return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)

    def layer_finish(self, d_ff, weights, h, attn_out, out, r_out=None, workspace=None, stream=None):
        """The rest of the layer in bf16: weights = (w_o, gamma, w_gate, w_up, w_down);
        out = bf16(r + bf16(swiglu(...) W_down^T)) with r = bf16(h + bf16(attn_out W_o^T))."""
        names = ("w_o", "gamma", "w_gate", "w_up", "w_down")
        for name, t in list(zip(names, weights)) + [("h", h), ("attn_out", attn_out), ("out", out)]:
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
        n, D = h.shape
        if out.shape != h.shape or attn_out.shape[0] != n or (r_out is not None and r_out.shape != h.shape):
            raise ValueError("h, out (and r_out) must be [n_rows, d_model], attn_out [n_rows, n_heads head_dim]")
        w = LayerWeights(*[t.data_ptr() for t in weights])
        ws = workspace if workspace is not None else self.layer_workspace(d_ff, n, r_out is not None, h.device)
        st = self.lib.lacache_layer_finish(self.handle, d_ff, ctypes.byref(w), _ptr(h), _ptr(attn_out), n,
                                           _ptr(r_out), _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
        self._check(st, "lacache_layer_finish")
        return ws

    def sampler_workspace(self, vocab, table, device="cuda"):
        n = ctypes.c_size_t()
        seqs = _seqs(table)
        self._check(self.lib.lacache_sampler_workspace_size(self.handle, vocab, seqs, len(table), ctypes.byref(n)),
                    "lacache_sampler_workspace_size")
        return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)

    def sampler_cut(self, hidden, table, gamma_f, w_lm, token, confidence, probs=None, workspace=None, stream=None):
        """Final norm, lm-head and float softmax of the block rows of `table`:
        token [M] int32 (argmax), confidence [M] fp32, probs [M, vocab] fp32 or None."""
        for name, t in (("hidden", hidden), ("gamma_f", gamma_f), ("w_lm", w_lm)):
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
        if token.dtype != torch.int32 or confidence.dtype != torch.float32:
            raise ValueError("token must be int32 and confidence fp32")
        vocab = w_lm.shape[0]
        M = sum(be - bs for _, _, bs, be in table)
        if token.numel() < M or confidence.numel() < M or (probs is not None and probs.numel() < M * vocab):
            raise ValueError("token / confidence / probs are smaller than the block rows")
        seqs = _seqs(table)
        ws = workspace if workspace is not None else self.sampler_workspace(vocab, table, hidden.device)
        st = self.lib.lacache_sampler_cut(self.handle, _ptr(hidden), hidden.shape[0], seqs, len(table), _ptr(gamma_f),
                                          _ptr(w_lm), vocab, _ptr(token), _ptr(confidence), _ptr(probs), _ptr(ws),
                                          ws.numel(), _stream(stream))
        self._check(st, "lacache_sampler_cut")
        return ws

    # ------------------------------------------------------------------
    # Selective cache update and two-view verify
    # ------------------------------------------------------------------
    def track_workspace(self, n_rows, device="cuda"):
        n = ctypes.c_size_t()
        self._check(self.lib.lacache_track_workspace_size(self.handle, n_rows, ctypes.byref(n)),
                    "lacache_track_workspace_size")
        return torch.empty(max(n.value, 256), dtype=torch.uint8, device=device)

    def track_select(self, ct: CacheTensors, table, budget, importance, tracked, workspace=None, stream=None):
        """Importance of every row (importance [n_rows] fp32) for the block queries in ct.q with the LSE in
        ct.lse, and the tracking set (tracked [batch, budget] int32, positions within the sample, -1 pads)."""
        if importance.dtype != torch.float32 or tracked.dtype != torch.int32:
            raise ValueError("importance must be fp32 and tracked int32")
        if importance.numel() < ct.n_rows or tracked.numel() < len(table) * budget:
            raise ValueError("importance or tracked is too small")
        ws = workspace if workspace is not None else self.track_workspace(ct.n_rows, importance.device)
        cache = self._cache(ct)
        st = self.lib.lacache_track_select(self.handle, ctypes.byref(cache), _ptr(ct.lse), _seqs(table), len(table),
                                          budget, _ptr(importance), _ptr(tracked), _ptr(ws), ws.numel(),
                                          _stream(stream))
        self._check(st, "lacache_track_select")

    def verify_attn(self, q_ver, k_ver, v_ver, view, pos, ver_start, ct: CacheTensors, table, out, lse=None,
                    stream=None):
        """Two-view verify attention; ver_start: host list [batch + 1] of the samples' first verify tokens."""
        for name, t in (("q_ver", q_ver), ("k_ver", k_ver), ("v_ver", v_ver)):
            if t.dtype != torch.float16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous fp16 CUDA tensor")
        if view.dtype != torch.int32 or pos.dtype != torch.int32 or out.dtype != torch.bfloat16:
            raise ValueError("view and pos must be int32, out bf16")
        starts = (ctypes.c_int32 * (len(table) + 1))(*[int(x) for x in ver_start])
        cache = self._cache(ct)
        st = self.lib.lacache_verify_attn(self.handle, _ptr(q_ver), _ptr(k_ver), _ptr(v_ver), _ptr(view), _ptr(pos),
                                         starts, ctypes.byref(cache), _seqs(table), len(table), _ptr(out), _ptr(lse),
                                         _stream(stream))
        self._check(st, "lacache_verify_attn")

    def verify_accept(self, draft, mask_tok, mask_conf, pos, search_start, table, gamma, ids, n_accepted,
                      stream=None):
        """Sequential acceptance; search_start: host list [batch + 1]; updates ids in place."""
        for name, t in (("draft", draft), ("mask_tok", mask_tok), ("pos", pos), ("ids", ids),
                        ("n_accepted", n_accepted)):
            if t.dtype != torch.int32 or not t.is_cuda:
                raise ValueError(f"{name} must be an int32 CUDA tensor")
        starts = (ctypes.c_int32 * (len(table) + 1))(*[int(x) for x in search_start])
        st = self.lib.lacache_verify_accept(self.handle, _ptr(draft), _ptr(mask_tok), _ptr(mask_conf), _ptr(pos),
                                           starts, _seqs(table), len(table), float(gamma), _ptr(ids),
                                           _ptr(n_accepted), _stream(stream))
        self._check(st, "lacache_verify_accept")

    def profile(self, enable: bool):
        """Bracket every launch with HIP events (diagnostics)."""
        self._check(self.lib.lacache_profile_enable(self.handle, int(bool(enable))), "lacache_profile_enable")

    def profile_read(self):
        """{kernel name: (total ms, launches)} since the last read; synchronises the events."""
        res = {}
        for k, name in enumerate(KERNEL_NAMES):
            ms, n = ctypes.c_double(), ctypes.c_int64()
            self._check(self.lib.lacache_profile_read(self.handle, k, ctypes.byref(ms), ctypes.byref(n)),
                        "lacache_profile_read")
            res[name] = (ms.value, n.value)
        return res

    def read_device_status(self, stream=None):
        flags = ctypes.c_uint32()
        self._check(self.lib.lacache_read_device_status(self.handle, _stream(stream), ctypes.byref(flags)),
                    "lacache_read_device_status")
        return flags.value


def context_for(wl, max_seq_len=None):
    """Context for a synthetic workload (exact_attention_state_amd.synth.Workload)."""
    return Context(wl.d_model, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.vocab,
                   max_seq_len or max(wl.seq_lens), wl.rope_theta, wl.rms_eps, 0.0, wl.dtype)
