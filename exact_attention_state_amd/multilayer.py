"""Approximate deeper-layer reuse on the GPU: a model of L transformer layers
of one shape, driven through the C ABI only (every step of the computation
runs in the library's kernels; this module orders the calls and holds the
buffers).

* ``refresh(ids)``: the full forward, every layer on every row.  Layer l
  reads its input rows X[l] as its "embedding table" with the row indices as
  ids, so the same projection kernels serve every layer; the refresh leaves
  each layer's RoPECache (and layer 0's FACache) exact for these ids.
* ``step(block_ids)``: one approximate inner step of block-wise decoding
  (the DualCache page, "Block-wise Generation"; LaCache Appendix C): layer 0
  exactly (LaCache's cached block step), then at every later layer only the
  block rows: their fresh q, k, v (lacache_project_block) attend over the
  layer's keys, the other rows' being those of the last refresh
  (lacache_dualcache_attn), and the rest of the layer runs on the block rows
  (lacache_layer_finish).  The other rows' inputs stay those of the refresh.
* ``run_block(ids_per_step, r)``: a block's inner steps with a refresh at the
  first step and every r steps after it (r = None: block boundary only; the
  DualCache page's refresh_interval).
"""

from __future__ import annotations

import numpy as np
import torch

from . import lacache


def _bf16(x, device):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(device)


class MultiLayer:
    def __init__(self, params, head_dim, d_ff, table, rope_theta=1e4, rms_eps=1e-5, device="cuda",
                 weights_from: "MultiLayer | None" = None):
        """params: host arrays (synth.multilayer_params); table: the block table
        [(seq_offset, seq_len, block_start, block_end)]; weights_from: another
        instance whose device weights this one shares."""
        self.table = [tuple(int(x) for x in s) for s in table]
        self.device = device
        E = params["embed"]
        D = E.shape[1]
        self.L = len(params["layers"])
        self.D, self.F, self.dh = D, d_ff, head_dim
        self.H = params["layers"][0]["w_qkv"].shape[0] // (3 * head_dim)
        self.HD = self.H * head_dim
        self.T = max(o + n for o, n, _, _ in self.table)
        max_len = max(n for _, n, _, _ in self.table)
        self.ctx0 = lacache.Context(D, self.H, self.H, head_dim, E.shape[0], max_len, rope_theta, rms_eps, 0.0, "bf16")
        self.ctxl = lacache.Context(D, self.H, self.H, head_dim, self.T, max_len, rope_theta, rms_eps, 0.0, "bf16")
        if weights_from is not None:
            self.E, self.qkv, self.lw = weights_from.E, weights_from.qkv, weights_from.lw
        else:
            self.E = _bf16(E, device)
            self.qkv, self.lw = [], []
            for li, lp in enumerate(params["layers"]):
                ctx = self.ctx0 if li == 0 else self.ctxl
                g, w = _bf16(lp["gamma_attn"], device), _bf16(lp["w_qkv"], device)
                self.qkv.append((g, w, ctx.pack_qkv_weight(w)))
                self.lw.append([_bf16(lp[k], device) for k in ("w_o", "gamma_ffn", "w_gate", "w_up", "w_down")])
        # X[l]: the input rows of layer l (X[L]: the model's output rows)
        self.X = [None] + [torch.zeros(self.T, D, dtype=torch.bfloat16, device=device) for _ in range(self.L)]
        self.ct = [(self.ctx0 if li == 0 else self.ctxl).alloc_cache(self.T, device) for li in range(self.L)]
        self.row_ids = torch.arange(self.T, dtype=torch.int32, device=device)
        self.block_rows = [slice(o + bs, o + be) for o, _, bs, be in self.table]
        self.block_row_ids = torch.from_numpy(
            np.concatenate([np.arange(s.start, s.stop) for s in self.block_rows]).astype(np.int32)).to(device)
        self.M = int(self.block_row_ids.numel())
        self.out_block = torch.empty(self.M, self.H, head_dim, dtype=torch.bfloat16, device=device)
        ws = lambda ctx, op, table: ctx.alloc_workspace(op, table, device)
        self.ws_prefill = [ws(self.ctx0, lacache.OP_PREFILL, self.table), ws(self.ctxl, lacache.OP_PREFILL, self.table)]
        self.ws_step = ws(self.ctx0, lacache.OP_BLOCK_STEP, self.table)
        self.ws_proj = ws(self.ctxl, lacache.OP_PROJECT_BLOCK, self.table)
        self.ws_dual = [ws(self.ctxl, lacache.OP_DUALCACHE_ATTN, [s]) for s in self.table]
        self.ws_layer = self.ctx0.layer_workspace(d_ff, self.T, False, device)   # r lives in the workspace

    def _weights(self, li):
        g, w, wp = self.qkv[li]
        emb = self.E if li == 0 else self.X[li]
        return (emb, g, w) if wp is None else (emb, g, w, wp)

    def refresh(self, ids, stream=None):
        """The full forward with ids [T] (device int32)."""
        T, HD = self.T, self.HD
        for li in range(self.L):
            ctx = self.ctx0 if li == 0 else self.ctxl
            ct = self.ct[li]
            ctx.prefill_cache(self._weights(li), ids if li == 0 else self.row_ids, self.table, ct,
                              workspace=self.ws_prefill[0 if li == 0 else 1], stream=stream)
            h = ct.h if li == 0 else self.X[li]
            ctx.layer_finish(self.F, self.lw[li], h, ct.out.view(T, HD), self.X[li + 1], workspace=self.ws_layer,
                             stream=stream)

    def step(self, block_ids, stream=None):
        """One approximate inner step with the blocks' new ids (device int32 [M])."""
        HD = self.HD
        ct0 = self.ct[0]
        self.ctx0.block_step(self._weights(0), block_ids, self.table, ct0, self.ws_step, stream=stream)
        for rows in self.block_rows:
            n = rows.stop - rows.start
            self.ctx0.layer_finish(self.F, self.lw[0], ct0.h[rows], ct0.out[rows].view(n, HD), self.X[1][rows],
                                   workspace=self.ws_layer, stream=stream)
        for li in range(1, self.L):
            ct = self.ct[li]
            self.ctxl.project_block(self._weights(li), self.block_row_ids, self.table, ct, workspace=self.ws_proj,
                                    stream=stream)
            r0 = 0
            for b, rows in enumerate(self.block_rows):
                n = rows.stop - rows.start
                ob = self.out_block[r0:r0 + n]
                self.ctxl.dualcache_attn(ct.q[rows], ct.k, ct.v, [self.table[b]], ob, workspace=self.ws_dual[b],
                                         stream=stream)
                self.ctxl.layer_finish(self.F, self.lw[li], self.X[li][rows], ob.view(n, HD), self.X[li + 1][rows],
                                       workspace=self.ws_layer, stream=stream)
                r0 += n

    def block_output(self):
        """The block rows of the last layer's output [M, D] (block-table order)."""
        return torch.cat([self.X[self.L][rows] for rows in self.block_rows])

    def run_block(self, steps, r, stream=None):
        """Steps of one block: refresh at step 0 and at every step k with r | k,
        approximate steps otherwise.  steps: per step (ids [T], block ids [M]),
        device int32.  Returns the block output after each step and which
        steps refreshed."""
        outs, refreshed = [], []
        for k, (ids, block_ids) in enumerate(steps):
            if k == 0 or (r is not None and k % r == 0):
                self.refresh(ids, stream)
                refreshed.append(True)
            else:
                self.step(block_ids, stream)
                refreshed.append(False)
            outs.append(self.block_output())
        return outs, refreshed
