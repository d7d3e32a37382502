"""fp64 CPU oracles: LaCache's exact layer-0 step (lacache_ref, re-exported
here), the per-group FP8 FFN of the later layers (fp8_ref), and the rest of
layer 0 with the sampler cut (layer_ref).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
Parity of the readings it shares with the HIP path (softmax scale, RoPE
pairing, RMSNorm eps) against a real LLaDA checkpoint is unpinned.
"""

from .lacache_ref import *  # noqa: F401,F403
from .lacache_ref import __all__  # noqa: F401
