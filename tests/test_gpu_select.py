"""GPU idx_select: bit-identical to idx_topk over the library's own scores (and the
column -> token map for candidate blocks), and end-to-end against the oracle under the
overlap / tie-gap rule; sparse-block selection equals the dense-masked selection."""
import numpy as np
import pytest

import dsa_lightning_indexer_idx_amd as D
import oracle as O
import synth
from full_cases import full_case
from gpu_util import record, Uploaded, assert_selection_matches, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_dense": lambda: synth.tiny_dense(),
    "dense_fp8_ragged": lambda: synth.batched_decode(seed=131, rows=5, n=6000, ragged=True, gap=33),
    "dense_mxfp4": lambda: synth.batched_decode(seed=132, rows=3, n=4000, kdtype="mxfp4"),
    "paged_fp8": lambda: synth.paged_decode(seed=133, rows=5, min_len=100, max_len=9000,
                                            row_req=True),
    "paged_mxfp4": lambda: synth.paged_decode(seed=134, rows=4, min_len=3000, max_len=6000,
                                              kdtype="mxfp4"),
    "sparse_mxfp4": lambda: synth.sparse_blocks(seed=135, rows=5, ctx=16384, n_blocks=24,
                                                ragged=True),
    "sparse_fp8": lambda: synth.sparse_blocks(seed=136, rows=3, ctx=8192, n_blocks=20,
                                              kdtype="fp8"),
    "prefill": lambda: synth.prefill_chunk(seed=137, q_tokens=96, prior=3000),
    "paged_sparse_mxfp4": lambda: synth.paged_sparse_blocks(seed=138, rows=5, ctx=16384, n_blocks=24, ragged=True,
                                                            row_req=True),
    "paged_sparse_fp8": lambda: synth.paged_sparse_blocks(seed=139, rows=3, ctx=8192, n_blocks=20, kdtype="fp8"),
}


def _self_consistent(up, k):
    """idx_select == idx_topk(idx_logits*) bit for bit."""
    case = up.case
    s_idx, s_val = up.select(k)
    lg = up.logits()
    if up.kind == "Dense":
        lens = up.ke - up.ks
    elif up.kind == "Paged":
        lens = up.sl
    else:
        lens = up.nc
    t_idx, t_val = D.idx_topk(lg, k, lens=lens.contiguous(), n_cols=lg.shape[1])
    t_idx, t_val = host(t_idx), host(t_val)
    if up.kind in ("Sparse", "PagedSparse"):
        t_idx = O.columns_to_tokens(t_idx, case.cand, case.block)
    s_idx, s_val = host(s_idx), host(s_val)
    assert np.array_equal(s_idx, t_idx), "select != topk(logits)"
    assert np.array_equal(s_val, t_val)
    return s_idx, s_val


def _ref_scores_fn(case, ref_lg):
    if type(case).__name__ not in ("Sparse", "PagedSparse"):
        return lambda r, idx: ref_lg[r][idx]
    # sparse: selected values are tokens; find their columns
    def f(r, toks):
        cols = []
        for t in toks:
            b = np.searchsorted(case.cand[r], t // case.block)
            cols.append(b * case.block + t % case.block)
        return ref_lg[r][np.array(cols)]
    return f


@pytest.mark.parametrize("name", sorted(SMALL))
def test_select_small(name):
    require_gpu()
    case = SMALL[name]()
    up = Uploaded(case)
    k = min(case.topk, 2048)
    s_idx, _ = _self_consistent(up, k)
    r_idx, r_val, r_lg = O.select_case(case, k=k, with_logits=True)
    kth = np.array([r_val[r][max(0, int((r_idx[r] >= 0).sum()) - 1)] for r in range(case.rows)])
    inter, total = assert_selection_matches(s_idx, r_idx, _ref_scores_fn(case, r_lg), kth, name)
    say(f"[select] {name}: overlap {inter}/{total}")


def test_sparse_equals_dense_masked_on_gpu():
    """The candidate-block route and the dense route with non-candidate tokens masked pick
    the same tokens (scores agree within tolerance, so compare under the overlap rule)."""
    require_gpu()
    sp = synth.sparse_blocks(seed=138, rows=4, ctx=4096, n_blocks=10, ragged=True,
                             poison_noncand=False)
    g_idx, _ = Uploaded(sp).select(300)
    dense = synth.Dense("dense_view", sp.q, "fp8", sp.w, sp.k, sp.k_scale, sp.k_dtype, sp.row_ks,
                        sp.row_ke, 300)
    d_lg = host(Uploaded(dense).logits(ld=4096))
    mask = np.zeros_like(d_lg, dtype=bool)
    for r in range(sp.rows):
        cols = np.arange(int(sp.n_cols[r]))
        toks = sp.cand[r][cols // 128] * 128 + cols % 128
        toks = toks[toks < sp.row_ke[r] - sp.row_ks[r]]
        mask[r, toks] = True
    masked = np.where(mask, d_lg, -np.inf).astype(np.float32)
    m_idx, _ = D.idx_topk(dev(masked), 300)
    assert np.array_equal(host(g_idx), host(m_idx))


def test_unsorted_select_same_set():
    require_gpu()
    case = synth.paged_decode(seed=139, rows=3, min_len=5000, max_len=9000)
    up = Uploaded(case)
    a, _ = up.select(1024)
    b, _ = up.select(1024, sorted=False)
    a, b = host(a), host(b)
    for r in range(3):
        assert sorted(a[r].tolist()) == sorted(b[r].tolist())


WORKLOAD_NAMES = {2: "batched decode 32x32K fp8", 3: "paged decode 128K fp8", 4: "prefill 4096x8192 fp8",
                  5: "two-level 64x8192 mxfp4", 6: "paged decode 128K mxfp4", 7: "two-level paged 64x8192 mxfp4"}


def _oracle_select(case, ks):
    """The oracle's selection at each k from one computation of its scores: {k: (idx, val)}
    (idx: key positions as idx_select returns them) and the scores."""
    _, _, lg = O.select_case(case, k=max(ks), with_logits=True)
    kind = type(case).__name__
    if kind == "Paged":
        lens = case.seq_lens
    elif kind in ("Sparse", "PagedSparse"):
        lens = case.n_cols
    else:
        lens = case.row_ke.astype(np.int64) - case.row_ks
    lens = np.clip(lens, 0, lg.shape[1]).astype(np.int32)
    out = {}
    for k in ks:
        idx, val = O.topk(lg, k, lens=lens)
        if kind in ("Sparse", "PagedSparse"):
            idx = O.columns_to_tokens(idx, case.cand, case.block)
        out[k] = (idx, val)
    return out, lg


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6, 7])
def test_full_size_select(cfg):
    """The workloads at full size through idx_select (the benchmark's call): every row
    equals idx_topk over idx_logits* bit for bit, and the oracle checks every row end to
    end (every 8th row of the prefill chunk, with the first and last)."""
    require_gpu()
    case, up = full_case(cfg)
    ks = [2048, 1024, 512] if cfg == 3 else [case.topk]
    rows = list(range(0, case.rows, 8)) + [case.rows - 1] if cfg == 4 else list(range(case.rows))
    sub = case if len(rows) == case.rows else O.subset_rows(case, rows)
    say(f"[select] full workload {cfg}: oracle over {len(rows)} rows")
    ref, r_lg = _oracle_select(sub, ks)
    for k in ks:
        say(f"[select] full workload {cfg} k={k}")
        s_idx, _ = _self_consistent(up, k)
        r_idx, r_val = ref[k]
        kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(len(rows))])
        inter, total = assert_selection_matches(s_idx[rows], r_idx, _ref_scores_fn(sub, r_lg), kth,
                                                f"workload {cfg} k={k}")
        worst = assert_selection_matches.worst
        record("select", WORKLOAD_NAMES[cfg], f"k={k} ovl {inter / max(total, 1):.5f}", 0.0, worst,
               f"{len(rows)}/{case.rows}")
        say(f"[select] full workload {cfg} k={k}: overlap {inter}/{total}, worst disagreement {worst:.3f} of limit")


def test_batched_decode_256_rows():
    """256 decode rows of 32768 fp8 keys each (rows with their own contexts, as many as a
    prefill chunk has tiles of): idx_select takes the row scan and the one-pass selection,
    equals idx_topk over idx_logits bit for bit and matches the oracle on every row."""
    require_gpu()
    case = synth.batched_decode(seed=7, rows=256)
    up = Uploaded(case)
    say("[select] batched decode 256 x 32768")
    s_idx, _ = _self_consistent(up, 2048)
    ref, r_lg = _oracle_select(case, [2048])
    r_idx, r_val = ref[2048]
    kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(case.rows)])
    inter, total = assert_selection_matches(s_idx, r_idx, _ref_scores_fn(case, r_lg), kth, "batched 256 x 32K")
    record("select", "batched decode 256x32K fp8", f"k=2048 ovl {inter / max(total, 1):.5f}", 0.0,
           assert_selection_matches.worst, f"{case.rows}/{case.rows}")


def test_long_rows_adversarial():
    """Rows of up to 131072 columns (the long-row top-k path) with adversarial content:
    equal scores everywhere (w = 0: the cut bin holds the whole row, more than the
    candidate lists keep, so the row is finished from itself), a short row among long
    ones, a row of tiny scores; each k equals idx_topk over the same scores bit for bit,
    and the oracle confirms the equal-score and short rows."""
    require_gpu()
    case = synth.paged_decode(seed=140, rows=8, min_len=40000, max_len=131072)
    case.w[1] = 0.0
    case.w[2] *= np.float32(1e-20)
    case.seq_lens[3] = 5000
    up = Uploaded(case)
    for k in (2048, 512, 64):
        say(f"[select] long adversarial rows k={k}")
        s_idx, _ = _self_consistent(up, k)
        rows = [1, 3]
        sub = O.subset_rows(case, rows)
        r_idx, r_val, r_lg = O.select_case(sub, k=k, with_logits=True)
        kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(len(rows))])
        assert_selection_matches(s_idx[rows], r_idx, _ref_scores_fn(sub, r_lg), kth, f"long rows k={k}")
        assert np.array_equal(s_idx[1], np.arange(k, dtype=np.int32)), "equal scores: the first k"


@pytest.mark.parametrize("shape", ["uniform", "ragged"])
def test_select_spilled_ranges(shape):
    """More steps than a workgroup keeps in LDS (about 600 per workgroup): the one-pass
    selection reads the spilled scores for its histogram and its filter, rows span two to
    several workgroups and share their histograms; every row equals idx_topk over
    idx_logits bit for bit and the oracle confirms sampled rows."""
    require_gpu()
    if shape == "uniform":
        case = synth.batched_decode(seed=151, rows=160, n=65536)
    else:
        case = synth.batched_decode(seed=152, rows=200, n=98304, ragged=True)
    up = Uploaded(case)
    lens = case.row_ke - case.row_ks
    rows = sorted({0, 1, case.rows // 2, case.rows - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    sub = O.subset_rows(case, rows)
    for k in (2048, 512):
        say(f"[select] spilled ranges {shape} k={k}")
        s_idx, _ = _self_consistent(up, k)
        r_idx, r_val, r_lg = O.select_case(sub, k=k, with_logits=True)
        kth = np.array([r_val[i][max(0, int((r_idx[i] >= 0).sum()) - 1)] for i in range(len(rows))])
        assert_selection_matches(s_idx[rows], r_idx, _ref_scores_fn(sub, r_lg), kth, f"spilled {shape} k={k}")
