"""The block step captured in a HIP graph and replayed (the launch path the
benchmark times), against the same step launched eagerly, bit for bit.
Replays alternate with eager steps on the same workspace and caches and with
unrelated eager work; every replay and every eager step must reproduce its
eager reference, and the device status must stay clear."""

import sys

import pytest
import torch

from exact_attention_state_amd import lacache, synth
from exact_attention_state_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["llada8b", "tiny_batched16"])
def test_step_graph_replays_match_eager(name):
    wl = synth.WORKLOADS[name]
    _say(f"[graph] {name}: batch {wl.batch}")
    dw = DeviceWorkload(wl, device="cuda")
    dw.prefill()
    blk = [dw.next_block_ids() for _ in range(2)]
    torch.cuda.synchronize()
    ref = []
    for b in blk:                                        # eager results of the two edit steps
        dw.block_step(b)
        torch.cuda.synchronize()
        ref.append((dw.ct.out.clone(), dw.ct.lse.clone()))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            dw.block_step(blk[1], stream=stream)
    torch.cuda.synchronize()
    for rep in range(4):
        dw.ct.out.fill_(0)
        dw.ct.lse.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.ct.out, ref[1][0]) and torch.equal(dw.ct.lse, ref[1][1]), f"replay {rep} differs"
        # an eager step on the same workspace in between, and unrelated work
        dw.block_step(blk[rep % 2])
        x = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.equal(dw.ct.out, ref[rep % 2][0]), f"eager step after replay {rep} differs"
        assert float(x) == float(x)
    assert dw.ctx.read_device_status() == 0
    _say(f"  4 replays equal to the eager step, eager steps between them equal too")
