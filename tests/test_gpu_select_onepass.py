"""GPU idx_select through the one-pass selection (rows that read their own keys: the scan
adds each group's largest score to its row's histogram, cuts at the k-th largest group
maximum and writes the entries above the cut for an exact finish), forced with
IDX_SELECT_ONE_PASS for the shorter rows the default sends to scores-then-top-k. Every result must equal
idx_topk over idx_logits* bit for bit, with the cutoff and without it, whatever the
workspace held before, on rows the cutoff cannot shrink (equal scores, rows shorter than k)
and on rows with empty or clamped ranges; the scores-then-top-k path (prefill chunks, more
than 512 rows) gets the same range checks."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import oracle as O
import synth
from gpu_util import Uploaded, assert_selection_matches, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _reference(up, k, sorted=True):
    """idx_topk over the library's own scores (and the column -> token map)."""
    lg = up.logits()
    if up.kind == "Dense":
        lens = (up.ke - up.ks).clamp(min=0)
    elif up.kind == "Paged":
        lens = up.sl
    else:
        lens = up.nc
    t_idx, t_val = D.idx_topk(lg, k, lens=lens.contiguous(), n_cols=lg.shape[1], sorted=sorted)
    t_idx, t_val = host(t_idx), host(t_val)
    if up.kind in ("Sparse", "PagedSparse"):
        t_idx = O.columns_to_tokens(t_idx, up.case.cand, up.case.block)
    return t_idx, t_val


def _select(up, k, **kw):
    """idx_select through the one-pass selection (forced for rows the default would send
    to scores-then-top-k), unless the caller says otherwise."""
    kw.setdefault("one_pass", True)
    idx, val = D.idx_select(up.problem(), k, **kw)
    return host(idx), host(val)


# at least 8 rows: fewer take scores then top-k
CASES = {
    "paged_fp8": lambda: synth.paged_decode(seed=201, rows=10, min_len=3000, max_len=40000),
    "paged_mxfp4": lambda: synth.paged_decode(seed=202, rows=9, min_len=2000, max_len=30000, kdtype="mxfp4"),
    "dense_fp8": lambda: synth.batched_decode(seed=203, rows=12, n=9000, ragged=True, gap=21),
    "dense_bf16": lambda: synth.tiny_dense(seed=204, n=5000, rows=8, topk=300),
    "sparse_mxfp4": lambda: synth.sparse_blocks(seed=205, rows=10, ctx=16384, n_blocks=24, ragged=True),
    "sparse_fp8": lambda: synth.sparse_blocks(seed=206, rows=8, ctx=8192, n_blocks=12, kdtype="fp8"),
    "paged_sparse_mxfp4": lambda: synth.paged_sparse_blocks(seed=216, rows=12, ctx=16384, n_blocks=20, ragged=True,
                                                            row_req=True),
    "paged_sparse_fp8": lambda: synth.paged_sparse_blocks(seed=217, rows=9, ctx=8192, n_blocks=14, kdtype="fp8"),
    # fewer steps than workgroups: most workgroups hold one step or none
    "paged_fp8_tiny_rows": lambda: synth.paged_decode(seed=214, rows=8, min_len=1, max_len=1200),
    # rows ragged far past the 64-step slice and around the workgroup ranges
    "paged_fp8_long": lambda: synth.paged_decode(seed=215, rows=16, min_len=1, max_len=131072),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_cutoff_and_no_cutoff_equal_topk(name):
    require_gpu()
    case = CASES[name]()
    up = Uploaded(case)
    for k in sorted({1, 64, 512, min(case.topk, 2048), 2048}):
        say(f"[one-pass] {name} k={k}")
        r_idx, r_val = _reference(up, k)
        for cutoff in (True, False):
            s_idx, s_val = _select(up, k, cutoff=cutoff)
            assert np.array_equal(s_idx, r_idx), f"{name} k={k} cutoff={cutoff}: indices differ"
            assert np.array_equal(s_val, r_val), f"{name} k={k} cutoff={cutoff}: values differ"
        u_idx, _ = _select(up, k, sorted=False)
        for r in range(case.rows):
            assert sorted(u_idx[r].tolist()) == sorted(r_idx[r].tolist()), f"{name} k={k} unsorted row {r}"


def test_garbage_workspace_and_back_to_back_calls():
    """The workspace's counters are never cleared by the library: a workspace full of
    0xFF bytes, then calls of different shapes one after another on it, all give the
    exact selection."""
    require_gpu()
    a = Uploaded(synth.paged_decode(seed=207, rows=9, min_len=1000, max_len=20000))
    b = Uploaded(synth.paged_decode(seed=208, rows=12, min_len=30000, max_len=50000))
    need = max(D.idx_select_workspace(a.problem(), 2048), D.idx_select_workspace(b.problem(), 2048))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for up, k in ((a, 2048), (b, 1024), (a, 700), (b, 2048), (a, 2048)):
        r_idx, r_val = _reference(up, k)
        s_idx, s_val = D.idx_select(up.problem(), k, workspace=ws, one_pass=True)
        assert np.array_equal(host(s_idx), r_idx) and np.array_equal(host(s_val), r_val)


def test_rows_the_cutoff_cannot_shrink():
    """Equal scores (w = 0: every group maximum is equal, so every entry survives and the
    finish selects from the survivor regions themselves), tiny scores, a short row, an
    empty row and a row shorter than k, next to ordinary long rows."""
    require_gpu()
    case = synth.paged_decode(seed=209, rows=8, min_len=20000, max_len=60000)
    case.w[1] = 0.0
    case.w[2] *= np.float32(1e-20)
    case.seq_lens[3] = 5000
    case.seq_lens[4] = 0
    case.seq_lens[5] = 100
    case.seq_lens[6] = 1
    up = Uploaded(case)
    for k in (2048, 512, 64):
        r_idx, r_val = _reference(up, k)
        for cutoff in (True, False):
            s_idx, s_val = _select(up, k, cutoff=cutoff)
            assert np.array_equal(s_idx, r_idx) and np.array_equal(s_val, r_val), f"k={k} cutoff={cutoff}"
        assert np.array_equal(r_idx[1], np.arange(k, dtype=np.int32)), "equal scores: the first k"
        assert np.all(r_idx[4] == -1)
        assert np.all(r_idx[5][100:] == -1) and np.all(r_idx[5][:min(k, 100)] >= 0)
    # the oracle confirms the equal-score and short rows end to end
    rows = [1, 3, 5]
    sub = O.subset_rows(case, rows)
    s_idx, _ = _select(up, 512)
    r_idx, r_val, r_lg = O.select_case(sub, k=512, with_logits=True)
    kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(len(rows))])
    assert_selection_matches(s_idx[rows], r_idx, lambda r, ix: r_lg[r][ix], kth, "short / equal rows")


def test_empty_and_clamped_ranges_one_pass():
    """A candidate-block row whose key range is empty while n_cols > 0 selects nothing
    (padding), like the oracle; a dense row whose row_ke passes n_keys is clamped."""
    require_gpu()
    sp = synth.sparse_blocks(seed=210, rows=8, ctx=4096, n_blocks=8, kdtype="mxfp4", poison_noncand=False)
    sp.row_ke = sp.row_ke.copy()
    sp.row_ke[2] = sp.row_ks[2]  # no keys, n_cols still 8 blocks
    up = Uploaded(sp)
    for cutoff in (True, False):
        s_idx, _ = _select(up, 300, cutoff=cutoff)
        assert np.all(s_idx[2] == -1), "an empty range selects nothing"
        r_idx, _ = _reference(up, 300)
        assert np.array_equal(s_idx, r_idx)
    r_idx, r_val = O.select_case(sp, k=300)
    assert np.all(r_idx[2] == -1)
    dense = synth.batched_decode(seed=211, rows=9, n=3000)
    dense.row_ke = dense.row_ke.copy()
    dense.row_ke[2] = dense.k.shape[0] + 500  # past the key array: clamped to n_keys
    up = Uploaded(dense)
    D.idx_device_errors()
    for cutoff in (True, False):
        s_idx, s_val = _select(up, 512, cutoff=cutoff)
        r_idx, r_val = _reference(up, 512)
        assert np.array_equal(s_idx, r_idx) and np.array_equal(s_val, r_val)
    assert D.idx_device_errors() & D.IDX_DEVERR_RANGE


def test_empty_and_clamped_ranges_two_pass():
    """The same range cases on the scores-then-top-k path: a prefill-sized dense call
    (>= 256 rows, the tiled kernel) with a row past n_keys, and more than 512
    candidate-block rows with an empty range; the top-k reads only what was scored."""
    require_gpu()
    pf = synth.prefill_chunk(seed=212, q_tokens=260, prior=300)
    pf.row_ke = pf.row_ke.copy()
    pf.row_ke[7] = pf.k.shape[0] + 100
    up = Uploaded(pf)
    s_idx, s_val = _select(up, 256)
    r_idx, r_val = _reference(up, 256)
    assert np.array_equal(s_idx, r_idx) and np.array_equal(s_val, r_val)
    sp = synth.sparse_blocks(seed=213, rows=520, ctx=1024, n_blocks=3, kdtype="fp8", poison_noncand=False)
    sp.row_ke = sp.row_ke.copy()
    sp.row_ke[5] = sp.row_ks[5]
    up = Uploaded(sp)
    s_idx, _ = _select(up, 128)
    r_idx, _ = _reference(up, 128)
    assert np.all(s_idx[5] == -1)
    assert np.array_equal(s_idx, r_idx)


@pytest.mark.parametrize("n, rows", [(131072, 48), (65536, 64), (131072, 63)])
def test_speculative_cut_too_high(n, rows):
    """Rows whose top k sits in one stretch of keys (scales 8x over the first 30% of the
    row): the workgroup part holding that stretch takes a speculative cut from its own
    histogram far above the row's cut and is filtered again at the row's cut, on the
    16-column maxima path (128K-wide rows, and k = 512) and on the plain filter (64K-wide
    rows at k = 2048 take groups of 8). A cold stretch (scales / 8 over the second half)
    gives parts whose speculative cut lies far below. With 63 rows of 128K each range of
    a 256-CU device holds 504 of the 512 steps LDS keeps: no room past the scores for the
    last part's histogram, which then takes the first part's place. Every row equals
    idx_topk over idx_logits bit for bit; the oracle confirms the hot and cold rows."""
    require_gpu()
    case = synth.batched_decode(seed=221 + rows, rows=rows, n=n)
    hot, cold = [0, 5, rows - 1], [3]
    for r in hot:
        s = int(case.row_ks[r])
        case.k_scale[s:s + (3 * n) // 10] *= np.float32(8)
    for r in cold:
        s = int(case.row_ks[r])
        case.k_scale[s + n // 2:s + n] /= np.float32(8)
    up = Uploaded(case)
    check = sorted(hot + cold)
    sub = O.subset_rows(case, check)
    for k in (2048, 512):
        say(f"[one-pass] speculative cut, {rows} x {n}, k={k}")
        s_idx, s_val = _select(up, k, one_pass=False)
        t_idx, t_val = _reference(up, k)
        assert np.array_equal(s_idx, t_idx), "select != topk(logits)"
        assert np.array_equal(s_val, t_val)
        r_idx, r_val, r_lg = O.select_case(sub, k=k, with_logits=True)
        kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(len(check))])
        assert_selection_matches(s_idx[check], r_idx, lambda i, idx: r_lg[i][idx], kth, f"speculative {n} k={k}")
