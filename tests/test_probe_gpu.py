"""The streaming-read probe (a measurement aid): runs through the C ABI and
leaves the sink alone when no thread's folded words equal the key (an
all-zero buffer folds to 0 everywhere)."""

import pytest
import torch

import int4_weight_only_w4a16_amd as w4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 8 << 20])
def test_read_probe_runs_and_leaves_the_sink(nbytes):
    print(f"read probe: {nbytes} bytes", flush=True)
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.full((1,), 12345, dtype=torch.int32, device="cuda:0")
    w4.w4a16_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 12345
