"""GPU checks of the measurement aid (the streaming-read probe)."""
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_read_probe_runs_and_leaves_the_buffer_alone():
    require_gpu()
    buf = torch.arange(1 << 22, dtype=torch.int32, device="cuda")  # 16 MiB
    before = buf.clone()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    D.idx_read_probe(buf, sink)
    D.idx_read_probe(buf[:4], sink)  # one 16-byte vector
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
