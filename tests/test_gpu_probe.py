"""The HBM read probe runs on a device buffer, leaves its sink alone for contents whose
checksum cannot reach the marker value (all zeros), and reads at a plausible rate."""
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_probe_runs():
    import torch
    from speculative_decoding_amd import medusa as M
    dev = torch.device("cuda:0")
    buf = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    M.medusa_hbm_read_probe(buf, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        M.medusa_hbm_read_probe(buf, sink)
    b.record()
    torch.cuda.synchronize()
    gbps = 5 * (256 << 20) / (a.elapsed_time(b) * 1e-3) / 1e9
    say(f"[probe] {gbps:.0f} GB/s over 256 MiB")
    assert int(sink.item()) == 0
    assert gbps > 100.0
