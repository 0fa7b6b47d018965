"""GPU: the streaming-read probe (moe_hbm_read_probe), the measurement helper
that gives the read bandwidth a plain kernel reaches.  It must read any
16-byte-multiple buffer, ragged against its grid, and leave its sink alone
when the data's XOR cannot equal its key (an all-zero buffer)."""
import pytest
import torch

import int4_routed_expert_softmax_amd as moe

from moe_harness import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (64 << 20, 1024), ((64 << 20) + 48, 300)])
def test_read_probe_reads_and_leaves_sink_alone(nbytes, blocks):
    say(f"read probe: {nbytes} B, {blocks} blocks")
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device=DEV)
    moe.moe_hbm_read_probe(buf, sink, blocks)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0


def test_read_probe_times_with_the_timing_hook():
    buf = torch.ones(256 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(2048 * 256, dtype=torch.int32, device=DEV)
    ev = ([torch.cuda.Event(enable_timing=True) for _ in range(3)],
          [torch.cuda.Event(enable_timing=True) for _ in range(3)])
    h = moe.moe_timing_arm("read_probe", *ev)
    for _ in range(3):
        moe.moe_hbm_read_probe(buf, sink, 2048)
    torch.cuda.synchronize()
    assert moe.moe_timing_disarm(h) == 3
    ms = [s.elapsed_time(e) for s, e in zip(*ev)]
    say(f"read probe 256 MiB: {['%.3f' % m for m in ms]} ms")
    assert all(m > 0 for m in ms)
