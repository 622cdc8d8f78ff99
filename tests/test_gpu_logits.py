"""GPU scores (idx_logits, idx_logits_paged, idx_logits_sparse_blocks) against the oracle,
element by element: small cases spanning several tiles with ragged tails, the five
workloads at full size on sampled rows, and edge cases."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import record, score_error_stats, Uploaded, assert_scores_close, host, require_gpu, say
from full_cases import full_case

pytestmark = pytest.mark.gpu


def _ref_logits(case, ld=None):
    kind = type(case).__name__
    if kind == "Dense":
        return O.logits_dense(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                              case.row_ks, case.row_ke, ld=ld or case.max_cols)
    if kind == "Paged":
        return O.logits_paged(case.q, case.q_dtype, case.w, case.k_pages, case.k_scale_pages,
                              case.k_dtype, case.block_table, case.seq_lens, case.row_req, ld=ld)
    if kind == "PagedSparse":
        return O.logits_paged_sparse(case.q, case.q_dtype, case.w, case.k_pages, case.k_scale_pages, case.k_dtype,
                                     case.block_table, case.seq_lens, case.cand, case.n_cols, case.block,
                                     row_req=case.row_req, ld=ld)
    return O.logits_sparse(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                           case.row_ks, case.row_ke, case.cand, case.n_cols, case.block, ld=ld)


def _as_prefill(case):
    case.meta["as_prefill"] = True
    return case


SMALL = {
    "tiny_dense_bf16_n4096": lambda: synth.tiny_dense(),
    "dense_fp8_ragged": lambda: synth.batched_decode(seed=102, rows=5, n=3000, ragged=True, gap=40),
    "dense_mxfp4_ragged": lambda: synth.batched_decode(seed=103, rows=4, n=2500, kdtype="mxfp4",
                                                       ragged=True, gap=17),
    "dense_bf16_ragged": lambda: synth.batched_decode(seed=104, rows=3, n=1000, kdtype="bf16",
                                                      ragged=True, gap=5),
    "paged_fp8_rowreq": lambda: synth.paged_decode(seed=105, rows=6, min_len=1, max_len=3000,
                                                   row_req=True),
    "paged_mxfp4": lambda: synth.paged_decode(seed=106, rows=5, min_len=100, max_len=2100,
                                              kdtype="mxfp4"),
    "paged_fp8_page128": lambda: synth.paged_decode(seed=107, rows=4, min_len=200, max_len=1500,
                                                    page=128),
    "sparse_mxfp4_ragged": lambda: synth.sparse_blocks(seed=108, rows=5, ctx=4096, n_blocks=7,
                                                       ragged=True),
    "sparse_fp8_ragged": lambda: synth.sparse_blocks(seed=109, rows=4, ctx=3000, n_blocks=5,
                                                     kdtype="fp8", ragged=True),
    "paged_sparse_fp8_rowreq": lambda: synth.paged_sparse_blocks(seed=120, rows=5, ctx=4096, n_blocks=7,
                                                                 kdtype="fp8", ragged=True, row_req=True),
    "paged_sparse_mxfp4_page128": lambda: synth.page_sparse(
        synth.sparse_blocks(seed=121, rows=4, ctx=4096, n_blocks=6, ragged=True), page=128, seed=121),
    "paged_sparse_mxfp4_block64": lambda: synth.paged_sparse_blocks(seed=122, rows=3, ctx=2048, n_blocks=9,
                                                                    block=64, ragged=True),
    "prefill_q300_prior700": lambda: synth.prefill_chunk(seed=110, q_tokens=300, prior=700),
    # 300 decode rows with disjoint ragged ranges: the row scan
    "dense_many_rows_disjoint": lambda: synth.batched_decode(seed=116, rows=300, n=700, ragged=True,
                                                             gap=9),
    # the same rows handed over as a prefill chunk: the tiled kernel walks the union of each
    # query block's ranges (slow, still exact)
    "dense_many_rows_disjoint_as_prefill": lambda: _as_prefill(synth.batched_decode(seed=116, rows=300, n=700,
                                                                                    ragged=True, gap=9)),
    "prefill_q1030_prior64": lambda: synth.prefill_chunk(seed=117, q_tokens=1030, prior=64),
    # no prior context: the first query blocks see fewer keys than one 64-key tile, and the
    # 260-key array ends in a 4-key tile (tile loads clamped to the last key)
    "prefill_q260_prior0": lambda: synth.prefill_chunk(seed=118, q_tokens=260, prior=0),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_scores_match_oracle(name):
    require_gpu()
    case = SMALL[name]()
    say(f"[scores] {name}: rows={case.rows} max_cols={case.max_cols}")
    g = host(Uploaded(case).logits())
    r = _ref_logits(case, ld=g.shape[1])
    err = assert_scores_close(g, r, name)
    say(f"[scores] {name}: max |err| = {err:.3g}")


@pytest.mark.parametrize("name", ["tiny_dense_bf16_n4096", "dense_bf16_ragged"])
def test_bf16_scores_within_the_fp32_rounding_bound(name):
    """bf16 keys: every product q_d k_d is exact in fp32, so a score can only be off by the
    fp32 rounding of its two sums, 128 products per head and 64 weighted heads: at most
    about 2^-24 (128 A + 65 A) with A = sum_j |w_j| sum_d |q_jd k_d| (standard bound for
    recursive summation, either order). The test allows 2^-24 * 256 A, far tighter than
    the 1e-2 absolute tolerance on scores that spread over about 0.06 here."""
    require_gpu()
    case = SMALL[name]()
    g = host(Uploaded(case).logits())
    r = _ref_logits(case, ld=g.shape[1])
    q = np.abs(O.decode_bf16(case.q).astype(np.float64)).reshape(case.rows, 64, 128)
    k = np.abs(O.decode_bf16(case.k).astype(np.float64)).reshape(-1, 128)
    w = np.abs(case.w.astype(np.float64)).reshape(case.rows, 64)
    worst = 0.0
    for row in range(case.rows):
        s0, s1 = int(case.row_ks[row]), int(case.row_ke[row])
        A = w[row] @ (q[row] @ k[s0:s1].T)  # [s1 - s0]
        tol = 2.0 ** -24 * 256 * A
        err = np.abs(g[row, :s1 - s0].astype(np.float64) - r[row, :s1 - s0])
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), f"{name}: row {row}: {(err > tol).sum()} scores past the fp32 bound"
    err, ratio = score_error_stats(g, r)
    record("scores", "tiny dense bf16" if name.startswith("tiny") else "dense bf16 ragged", "",
           err, ratio, f"{case.rows}/{case.rows}")
    record("bf16", "tiny dense bf16" if name.startswith("tiny") else "dense bf16 ragged", "fp32 bound ",
           err, worst, f"{case.rows}/{case.rows}")
    say(f"[scores] {name}: max err / fp32 rounding bound = {worst:.3f}")


def test_paged_identity_table_equals_contiguous_bitwise():
    """A paged call whose table lays the pages out in order gives exactly the contiguous
    call's scores (same kernel arithmetic, different addressing)."""
    require_gpu()
    dense = synth.batched_decode(seed=111, rows=3, n=64 * 20)
    n = 64 * 20
    pages = dense.k.reshape(3 * 20, 64, 128)
    scales = dense.k_scale.reshape(3 * 20, 64)
    bt = np.arange(60, dtype=np.int32).reshape(3, 20)
    lens = np.array([n, n - 5, 700], np.int32)
    dense.row_ke = (dense.row_ks + lens).astype(np.int32)
    paged = synth.Paged("paged_identity", dense.q, "fp8", dense.w, pages, scales, "fp8", 64, bt,
                        lens, None, 16)
    gd = host(Uploaded(dense).logits(ld=n))
    gp = host(Uploaded(paged).logits(ld=n))
    assert np.array_equal(gd, gp)


@pytest.mark.parametrize("kd", ["fp8", "mxfp4"])
def test_paged_sparse_equals_sparse_bitwise(kd):
    """Candidate blocks read through a permuted page table (with a row -> request map)
    give exactly the scores of the same blocks of contiguous rows: same kernel arithmetic,
    different addressing."""
    require_gpu()
    sp = synth.sparse_blocks(seed=123, rows=6, ctx=8192, n_blocks=11, kdtype=kd, ragged=True)
    ps = synth.page_sparse(sp, page=64, seed=123, row_req=True)
    a = host(Uploaded(sp).logits())
    b = host(Uploaded(ps).logits())
    assert np.array_equal(a, b)


def test_ld_not_multiple_of_tile_and_empty_rows():
    require_gpu()
    case = synth.batched_decode(seed=112, rows=4, n=900, ragged=False)
    case.row_ke = case.row_ks + np.array([900, 0, 1, 63], np.int32)
    g = host(Uploaded(case).logits(ld=1000))
    r = _ref_logits(case, ld=1000)
    assert_scores_close(g, r, "ragged ld=1000")
    assert np.all(np.isneginf(g[1]))


def test_sparse_rows_without_columns():
    require_gpu()
    case = synth.sparse_blocks(seed=113, rows=3, ctx=2048, n_blocks=4, kdtype="mxfp4",
                               poison_noncand=False)
    case.n_cols = np.array([0, 1, 4 * 128], np.int32)
    g = host(Uploaded(case).logits())
    r = _ref_logits(case, ld=g.shape[1])
    assert_scores_close(g, r, "sparse n_cols edge")
    assert np.all(np.isneginf(g[0])) and np.isfinite(g[1, 0]) and np.all(np.isneginf(g[1, 1:]))


def test_bad_device_metadata_is_clamped_and_reported():
    """Out-of-range device values never fault: they are clamped and flagged."""
    require_gpu()
    import dsa_lightning_indexer_idx_amd as D
    D.idx_device_errors()
    case = synth.paged_decode(seed=114, rows=3, min_len=100, max_len=500, poison=False)
    case.block_table = case.block_table.copy()
    case.block_table[1, 0] = 10 ** 6
    up = Uploaded(case)
    g = host(up.logits())
    assert D.idx_device_errors() & D.IDX_DEVERR_PAGE
    r = _ref_logits(synth.paged_decode(seed=114, rows=3, min_len=100, max_len=500, poison=False),
                    ld=g.shape[1])
    assert_scores_close(g[[0, 2]], r[[0, 2]], "unaffected rows")
    dense = synth.batched_decode(seed=115, rows=2, n=300)
    dense.row_ke = dense.row_ke.copy()
    dense.row_ke[1] = dense.k.shape[0] + 1000
    host(Uploaded(dense).logits(ld=2000))
    assert D.idx_device_errors() & D.IDX_DEVERR_RANGE
    assert D.idx_device_errors() == 0


def test_candidate_block_checks_are_reported():
    """Candidate lists as the two-level path hands them over (ascending, unique, inside the
    row) raise no device error; a repeated block or a descending pair sets
    IDX_DEVERR_ORDER, a block past the row's range IDX_DEVERR_BLOCK (its columns scored
    -inf, like the oracle), and the other rows still match the oracle."""
    require_gpu()
    import dsa_lightning_indexer_idx_amd as D
    case = synth.sparse_blocks(seed=119, rows=4, ctx=4096, n_blocks=6, kdtype="fp8", poison_noncand=False)
    D.idx_device_errors()
    host(Uploaded(case).logits())
    assert D.idx_device_errors() == 0, "well-formed candidate lists"
    for what, edit, bit in (("repeated", lambda c: c.__setitem__((1, 3), c[1, 2]), D.IDX_DEVERR_ORDER),
                            ("descending", lambda c: c.__setitem__((1, slice(2, 4)), c[1, 2:4][::-1].copy()),
                             D.IDX_DEVERR_ORDER),
                            ("past the row", lambda c: c.__setitem__((1, 5), 4096 // case.block + 3),
                             D.IDX_DEVERR_BLOCK)):
        bad = synth.sparse_blocks(seed=119, rows=4, ctx=4096, n_blocks=6, kdtype="fp8", poison_noncand=False)
        bad.cand = bad.cand.copy()
        edit(bad.cand)
        g = host(Uploaded(bad).logits())
        assert D.idx_device_errors() & bit, what
        r = _ref_logits(bad, ld=g.shape[1])
        assert_scores_close(g, r, f"candidate lists, {what}")


WORKLOAD_NAMES = {2: "batched decode 32x32K fp8", 3: "paged decode 128K fp8", 4: "prefill 4096x8192 fp8",
                  5: "two-level 64x8192 mxfp4", 6: "paged decode 128K mxfp4", 7: "two-level paged 64x8192 mxfp4"}


def full_rows(cfg, rows):
    """Every row of the workload, or every 8th row (rows 0 and 4095 included) of the prefill
    chunk."""
    return list(range(0, rows, 8)) + [rows - 1] if cfg == 4 else list(range(rows))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6, 7])
def test_full_size_every_row(cfg):
    """The workloads at their stated sizes, in the launch shape the benchmark uses; the oracle
    checks every row (every 8th of the prefill chunk, with the first and last)."""
    require_gpu()
    case, up = full_case(cfg)
    say(f"[scores] full workload {cfg}: rows={case.rows} tokens={case.tokens}")
    g = host(up.logits())
    rows = full_rows(cfg, case.rows)
    sub = case if len(rows) == case.rows else O.subset_rows(case, rows)
    r = _ref_logits(sub, ld=g.shape[1])
    assert_scores_close(g[rows], r, f"workload {cfg}")
    err, ratio = score_error_stats(g[rows], r)
    record("scores", WORKLOAD_NAMES[cfg], "", err, ratio, f"{len(rows)}/{case.rows}")
    say(f"[scores] full workload {cfg}: {len(rows)} rows, max |err| = {err:.3g}, max err/tol = {ratio:.3f}")
