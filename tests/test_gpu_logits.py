"""GPU scores (idx_logits, idx_logits_paged, idx_logits_sparse_blocks) against the oracle,
element by element: small cases spanning several tiles with ragged tails, the five
workloads at full size on sampled rows, and edge cases."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import Uploaded, assert_scores_close, host, require_gpu, say
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
    return O.logits_sparse(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                           case.row_ks, case.row_ke, case.cand, case.n_cols, case.block, ld=ld)


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
    "prefill_q300_prior700": lambda: synth.prefill_chunk(seed=110, q_tokens=300, prior=700),
    # 300 rows take the tiled prefill kernel even though their ranges are disjoint and ragged
    "dense_many_rows_disjoint": lambda: synth.batched_decode(seed=116, rows=300, n=700, ragged=True,
                                                             gap=9),
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


FULL_SAMPLES = {2: [0, 17, 31], 3: [0, 40, 63], 4: [0, 1, 2047, 4095], 5: [0, 31, 63], 6: [0, 22, 63]}


@pytest.mark.parametrize("cfg", [2, 3, 4, 5, 6])
def test_full_size_sampled_rows(cfg):
    """The workloads at their stated sizes, in the launch shape the benchmark uses; the oracle
    checks a sample of rows."""
    require_gpu()
    case, up = full_case(cfg)
    say(f"[scores] full workload {cfg}: rows={case.rows} tokens={case.tokens}")
    g = host(up.logits())
    rows = FULL_SAMPLES[cfg]
    sub = O.subset_rows(case, rows)
    r = _ref_logits(sub, ld=g.shape[1])
    err = assert_scores_close(g[rows], r, f"workload {cfg}")
    say(f"[scores] full workload {cfg}: sampled rows {rows} max |err| = {err:.3g}")
