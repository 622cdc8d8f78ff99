"""GPU checks of the measurement aid (the streaming-read probe) and of the binding's
argument checks on device tensors."""
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


def test_binding_rejects_wrong_sizes_before_any_launch():
    """Sizes, dtypes and output shapes are checked in the binding: a tensor smaller than
    its role would otherwise be read or written out of bounds by the kernels."""
    require_gpu()
    dev = dict(device="cuda")
    q = torch.zeros((2, 64, 128), dtype=torch.uint8, **dev)
    w = torch.zeros((2, 64), dtype=torch.float32, **dev)
    k = torch.zeros((256, 128), dtype=torch.uint8, **dev)
    sc = torch.ones(256, dtype=torch.float32, **dev)
    ks = torch.zeros(2, dtype=torch.int32, **dev)
    ke = torch.full((2,), 256, dtype=torch.int32, **dev)
    with pytest.raises(ValueError, match="q has"):
        D.idx_logits(torch.zeros((2, 32, 128), dtype=torch.uint8, **dev), w, k, sc, ks, ke, k_dtype="fp8", ld=256)
    with pytest.raises(ValueError, match="contiguous"):
        D.idx_logits(q[:, :, ::2], w, k, sc, ks, ke, k_dtype="fp8", ld=256)
    with pytest.raises(ValueError, match="k_scale has"):
        D.idx_logits(q, w, k, sc[:128], ks, ke, k_dtype="fp8", ld=256)
    with pytest.raises(TypeError, match="row_ks"):
        D.idx_logits(q, w, k, sc, ks.long(), ke, k_dtype="fp8", ld=256)
    with pytest.raises(ValueError, match="out must be"):
        D.idx_logits(q, w, k, sc, ks, ke, k_dtype="fp8", out=torch.empty((1, 256), dtype=torch.float32, **dev))
    lg = torch.zeros((2, 256), dtype=torch.float32, **dev)
    with pytest.raises(ValueError, match="out_idx must be"):
        D.idx_topk(lg, 8, out_idx=torch.empty((2, 4), dtype=torch.int32, **dev))
    with pytest.raises(ValueError, match="lens has"):
        D.idx_topk(lg, 8, lens=torch.zeros(1, dtype=torch.int32, **dev))
    p = D.dense_problem(q, w, k, sc, ks, ke, k_dtype="fp8", max_cols=256)
    with pytest.raises(ValueError, match="out_idx must be"):
        D.idx_select(p, 8, out_idx=torch.empty((3, 8), dtype=torch.int32, **dev))
    qa = torch.zeros((2, 64, 576), dtype=torch.bfloat16, **dev)
    kv = torch.zeros((4, 64, 576), dtype=torch.bfloat16, **dev)
    bt = torch.zeros((2, 4), dtype=torch.int32, **dev)
    sl = torch.full((2,), 10, dtype=torch.int32, **dev)
    ix = torch.zeros((2, 16), dtype=torch.int32, **dev)
    with pytest.raises(ValueError, match="out has"):
        D.idx_sparse_attn_paged(qa, kv, bt, sl, ix, 0.1, out=torch.empty((2, 64, 256), dtype=torch.float32, **dev))
    with pytest.raises(ValueError, match="indices must have"):
        D.idx_sparse_attn_paged(qa, kv, bt, sl, ix[:1], 0.1)
    torch.cuda.synchronize()


def test_dispatch_log_lines():
    """IDX_LOG=1: each distinct dispatch decision is printed once to stderr (checked in a
    child process, since the setting is read once per process)."""
    require_gpu()
    import os
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})\n"
        "import synth, torch\n"
        "from gpu_util import Uploaded\n"
        "up = Uploaded(synth.paged_decode(seed=401, rows=12, min_len=20000, max_len=40000))\n"
        "for _ in range(3): up.select(512)\n"
        "up = Uploaded(synth.paged_decode(seed=402, rows=2, min_len=1000, max_len=9000))\n"
        "up.select(512); up.logits()\n"
        "torch.cuda.synchronize()\n"
    ).format(root=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
             tests=os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, IDX_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[dsaidx]")]
    assert sum("idx_select: one pass" in l for l in lines) == 1, lines
    assert any("idx_select: scan then top-k" in l for l in lines), lines
    assert any(l.startswith("[dsaidx] idx_logits_paged: balanced scan") for l in lines), lines
