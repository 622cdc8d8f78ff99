"""The entry points under HIP graph capture: each graph is replayed several times, with
eager work and synchronisations between replays, and every replay must reproduce the
eager result (the library records no memset nodes: its zeroing is done by kernels)."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import synth
from gpu_util import Uploaded, dev, host, require_gpu

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    fn()  # warm (one-time attribute setup happens outside the capture)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.capture_begin()
        fn()
        g.capture_end()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outs, want, disturb):
    for rep in range(4):
        for o in outs:
            o.fill_(7)           # stale contents must be overwritten
        disturb(rep)             # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), f"replay {rep} differs from the eager result"


def test_select_long_rows_under_capture():
    """Paged rows longer than 16384 columns: the scan clears the top-k histogram and the
    long-row kernels run; the workspace keeps the previous replay's contents."""
    require_gpu()
    case = synth.paged_decode(seed=151, rows=5, min_len=17000, max_len=40000, poison=False)
    up = Uploaded(case)
    p = up.problem()
    ws = torch.empty(D.idx_select_workspace(p, 1024), dtype=torch.uint8, device="cuda")
    oi = torch.empty((case.rows, 1024), dtype=torch.int32, device="cuda")
    ov = torch.empty((case.rows, 1024), dtype=torch.float32, device="cuda")
    D.idx_select(p, 1024, out_idx=oi, out_val=ov, workspace=ws)
    torch.cuda.synchronize()
    want = (oi.clone(), ov.clone())
    g = _capture(lambda: D.idx_select(p, 1024, out_idx=oi, out_val=ov, workspace=ws))
    noise = torch.empty_like(ws)
    _replays_match(g, (oi, ov), want, lambda rep: ws.copy_(noise.fill_(rep * 37 % 256)))


def test_prefill_select_under_capture():
    """A prefill chunk of 300 queries (the tiled prefill kernel, whose key tiles go from
    memory straight into LDS, then the short-row top-k) replayed from a graph."""
    require_gpu()
    case = synth.prefill_chunk(seed=153, q_tokens=300, prior=900, topk=512)
    up = Uploaded(case)
    p = up.problem()
    ws = torch.empty(D.idx_select_workspace(p, 512), dtype=torch.uint8, device="cuda")
    oi = torch.empty((case.rows, 512), dtype=torch.int32, device="cuda")
    ov = torch.empty((case.rows, 512), dtype=torch.float32, device="cuda")
    D.idx_select(p, 512, out_idx=oi, out_val=ov, workspace=ws)
    torch.cuda.synchronize()
    want = (oi.clone(), ov.clone())
    g = _capture(lambda: D.idx_select(p, 512, out_idx=oi, out_val=ov, workspace=ws))
    _replays_match(g, (oi, ov), want, lambda rep: ws.fill_(rep * 53 % 256))


def test_topk_and_short_rows_under_capture():
    require_gpu()
    rng = np.random.default_rng(152)
    lg_long = dev((rng.integers(-500, 500, (3, 40000)) / 8).astype(np.float32))
    lg_short = dev(rng.standard_normal((7, 5000)).astype(np.float32))
    lens = dev(np.array([40000, 20001, 123], np.int32))
    ws = torch.empty(D.lib().idx_topk_workspace(3, 40000, 2048), dtype=torch.uint8, device="cuda")
    a = D.idx_topk(lg_long, 2048, lens=lens, workspace=ws)
    b = D.idx_topk(lg_short, 300)
    torch.cuda.synchronize()
    want = [t.clone() for t in (*a, *b)]
    outs = [torch.empty_like(t) for t in want]

    def run():
        D.idx_topk(lg_long, 2048, lens=lens, workspace=ws, out_idx=outs[0], out_val=outs[1])
        D.idx_topk(lg_short, 300, out_idx=outs[2], out_val=outs[3])
    g = _capture(run)
    _replays_match(g, outs, want, lambda rep: ws.fill_(rep + 1))


def test_kcache_write_under_capture():
    require_gpu()
    rng = np.random.default_rng(153)
    keys = dev(synth.to_bf16_bits(rng.standard_normal((300, 128)).astype(np.float32))).view(torch.bfloat16)
    slots = dev(rng.permutation(512)[:300].astype(np.int64))
    cache = torch.zeros((512, 64), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((512, 4), dtype=torch.uint8, device="cuda")
    D.idx_kcache_write(keys, slots, cache, sc, "mxfp4")
    torch.cuda.synchronize()
    want = (cache.clone(), sc.clone())
    g = _capture(lambda: D.idx_kcache_write(keys, slots, cache, sc, "mxfp4"))
    written = torch.zeros(512, dtype=torch.bool, device="cuda")
    written[slots] = True
    for rep in range(4):
        cache.fill_(7)
        sc.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache[written], want[0][written]) and torch.equal(sc[written], want[1][written]), \
            f"replay {rep}: written slots differ"
        assert bool((cache[~written] == 7).all()) and bool((sc[~written] == 7).all()), \
            f"replay {rep}: a slot outside the mapping was written"
