"""GPU idx_candidate_blocks against the oracle, bit for bit: the published block ids and
counts for Gaussian and adversarial score rows (ties between block maxima, constant rows,
signed zeros, masked stretches, NaN holes, short and empty rows, huge magnitudes), over
block sizes, n_top values, both load paths (16-byte rows and unaligned ones), with and
without row lengths, at the long-decode source layer's full size, and under graph replay."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import oracle as O
import synth
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _check(lg, block, n_top, lens=None, what="", lg_dev=None):
    say(f"candidate blocks: {what} rows={lg.shape[0]} cols={lg.shape[1]} block={block} n_top={n_top}")
    g_c, g_n = D.idx_candidate_blocks(dev(lg) if lg_dev is None else lg_dev, block, n_top, lens=dev(lens))
    torch.cuda.synchronize()
    r_c, r_n = O.candidate_blocks(lg, block, n_top, lens)
    g_c, g_n = host(g_c), host(g_n)
    assert np.array_equal(g_n, r_n), f"{what}: counts differ at rows {np.flatnonzero(g_n != r_n)[:5]}"
    bad = np.argwhere(g_c != r_c)
    assert bad.size == 0, f"{what}: first mismatch at {bad[:3].tolist()}"


@pytest.mark.parametrize("block,n_top", [(128, 64), (64, 1), (64, 200), (256, 16), (1024, 8), (4096, 3),
                                         (192, 40)])
def test_small_mixed_rows(block, n_top):
    require_gpu()
    c = synth.candidate_scores(seed=70, rows=24, min_len=1, max_len=20000, ld=20004, block=block, n_top=n_top,
                               adversarial=True)
    _check(c.logits, block, n_top, c.lens, what="adversarial")
    g = synth.candidate_scores(seed=71, rows=9, min_len=3000, max_len=20000, ld=20004, block=block, n_top=n_top)
    _check(g.logits, block, n_top, g.lens, what="gaussian")


def test_unaligned_rows_and_no_lengths():
    """ld not a multiple of 4 and a start off a 16-byte boundary take the scalar-load
    path; lens=None scores every column."""
    require_gpu()
    c = synth.candidate_scores(seed=72, rows=16, min_len=1000, max_len=9999, ld=9999, block=128, n_top=20,
                               adversarial=True)
    _check(c.logits, 128, 20, c.lens, what="ld 9999")
    big = np.zeros((16, 10004), np.float32)
    big[:, 1:] = synth.candidate_scores(seed=73, rows=16, min_len=10003, max_len=10003, ld=10003).logits
    t = dev(big)
    view = t[:, 1:]                                   # rows start 4 bytes past a 16-byte boundary
    assert view.data_ptr() % 16 == 4
    say("candidate blocks: unaligned view")
    g_c, g_n = D.idx_candidate_blocks(view, 128, 32)
    r_c, r_n = O.candidate_blocks(big[:, 1:], 128, 32)
    assert np.array_equal(host(g_c), r_c) and np.array_equal(host(g_n), r_n)
    _check(big[:, 1:10001].copy(), 64, 50, None, what="no lengths")


def test_empty_and_tiny():
    require_gpu()
    lg = np.full((3, 64), -np.inf, np.float32)
    _check(lg, 64, 4, np.array([0, 64, 10], np.int32), what="all absent")
    lg = np.array([[0.5, -1.0, 2.0]], np.float32)
    _check(lg, 64, 2, None, what="three columns")
    say("candidate blocks: zero columns")
    e = torch.empty((2, 1), dtype=torch.float32, device="cuda")
    g_c, g_n = D.idx_candidate_blocks(e, 128, 5, n_cols=0)
    assert host(g_n).tolist() == [0, 0] and np.all(host(g_c) == -1)


def test_positions_past_n_top_untouched():
    require_gpu()
    c = synth.candidate_scores(seed=74, rows=8, min_len=2000, max_len=8000, ld=8192, block=128, n_top=12)
    cand = torch.full((8, 20), 777, dtype=torch.int32, device="cuda")
    say("candidate blocks: cand_ld 20, n_top 12")
    D.idx_candidate_blocks(dev(c.logits), 128, 12, lens=dev(c.lens), cand=cand)
    got = host(cand)
    r_c, _ = O.candidate_blocks(c.logits, 128, 12, c.lens)
    assert np.array_equal(got[:, :12], r_c)
    assert np.all(got[:, 12:] == 777)


def test_full_size_long_decode_source():
    """64 rows x 131072 columns, lengths of the long paged decode (U{65536..131072}),
    128-token blocks, 64 published per row."""
    require_gpu()
    c = synth.candidate_scores()
    _check(c.logits, c.block, c.n_top, c.lens, what="full size")
    a = synth.candidate_scores(seed=75, adversarial=True)
    _check(a.logits, a.block, a.n_top, a.lens, what="full size adversarial")


def test_graph_replay_matches_eager():
    """Captured once, replayed several times with eager work between: every replay
    gives the eager result."""
    require_gpu()
    c = synth.candidate_scores(seed=76, rows=32, min_len=4000, max_len=60000, ld=60000, block=128, n_top=64,
                               adversarial=True)
    lg, ln = dev(c.logits), dev(c.lens)
    cand = torch.empty((32, 64), dtype=torch.int32, device="cuda")
    n_cand = torch.empty(32, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(D.idx_candidate_blocks_workspace(32, 60000), 1), dtype=torch.uint8, device="cuda")
    say("candidate blocks: eager")
    D.idx_candidate_blocks(lg, 128, 64, lens=ln, cand=cand, n_cand=n_cand, workspace=ws)
    torch.cuda.synchronize()
    want_c, want_n = host(cand).copy(), host(n_cand).copy()
    r_c, r_n = O.candidate_blocks(c.logits, 128, 64, c.lens)
    assert np.array_equal(want_c, r_c) and np.array_equal(want_n, r_n)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    say("candidate blocks: capture")
    with torch.cuda.stream(s):
        D.idx_candidate_blocks(lg, 128, 64, lens=ln, cand=cand, n_cand=n_cand, workspace=ws, stream=s)
        torch.cuda.synchronize()
        g.capture_begin()
        D.idx_candidate_blocks(lg, 128, 64, lens=ln, cand=cand, n_cand=n_cand, workspace=ws, stream=s)
        g.capture_end()
    torch.cuda.synchronize()
    for i in range(4):
        cand.fill_(-5)
        n_cand.fill_(-5)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        say(f"candidate blocks: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(cand), want_c) and np.array_equal(host(n_cand), want_n), f"replay {i}"


@pytest.mark.parametrize("block,n_cols", [(64, 131072), (128, 300000), (4096, 4096 * 1500)])
def test_rows_of_more_than_1024_blocks(block, n_cols):
    """Rows past 1024 blocks take the workgroup selection (keys in LDS, radix select)."""
    require_gpu()
    rows = 8 if n_cols <= 300000 else 1
    c = synth.candidate_scores(seed=77, rows=rows, min_len=n_cols // 2, max_len=n_cols, ld=n_cols, block=block,
                               n_top=100, adversarial=rows > 1)
    _check(c.logits, block, 100, c.lens, what=f"{n_cols} columns")
