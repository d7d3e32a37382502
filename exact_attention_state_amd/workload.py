"""Device-side plumbing for a synthetic workload: upload parameters and ids,
allocate caches and workspaces, run the refresh and the inner steps through
the C ABI.  PyTorch is used for device memory and streams only.
"""

from __future__ import annotations

import numpy as np
import torch

from . import lacache, synth


def to_device_array(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 array (exactly representable in `dtype`) -> device tensor of that dtype."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(a if a.flags.writeable else a.copy())
    if dtype == "bf16":
        t = t.to(torch.bfloat16)          # exact: values are bf16-representable
    return t.to(device)


class DeviceWorkload:
    """Parameters, ids, caches and workspace of one synthetic workload on the GPU."""

    def __init__(self, wl: synth.Workload, device="cuda", ctx: lacache.Context | None = None, n_rows=None,
                 packed=True):
        """packed: also hand the library the packed fp16 projection weight (where the configuration has one)."""
        self.wl = wl
        self.device = device
        p = synth.params(wl)
        self.params = p
        self.weights = tuple(to_device_array(p[k], wl.dtype, device) for k in ("embed", "gamma", "w_qkv"))
        self.ctx = ctx or lacache.context_for(wl)
        if packed:
            wp = self.ctx.pack_qkv_weight(self.weights[2])
            if wp is not None:
                self.weights = self.weights + (wp,)
        self.table = wl.table()
        self.n_rows = n_rows or wl.total_tokens
        self.ct = self.ctx.alloc_cache(self.n_rows, device)
        self.ws = self.ctx.alloc_workspace(lacache.OP_BLOCK_STEP, self.table, device)
        self.ids_host = synth.initial_ids(wl)
        self.step = 0

    def upload_ids(self, ids_host):
        t = torch.zeros(self.n_rows, dtype=torch.int32)
        t[: len(ids_host)] = torch.from_numpy(np.asarray(ids_host, dtype=np.int32))
        return t.to(self.device)

    def prefill(self, stream=None):
        ws = self.ctx.alloc_workspace(lacache.OP_PREFILL, self.table, self.device)
        self.ctx.prefill_cache(self.weights, self.upload_ids(self.ids_host), self.table, self.ct, workspace=ws,
                               stream=stream)

    def next_block_ids(self):
        """Advance the host ids by one edit step; returns the device block ids."""
        self.step += 1
        self.ids_host, blk = synth.step_ids(self.wl, self.ids_host, self.step)
        return torch.from_numpy(blk).to(self.device)

    def block_step(self, block_ids, stream=None):
        self.ctx.block_step(self.weights, block_ids, self.table, self.ct, self.ws, stream=stream)
