"""Helpers for the GPU parity tests: upload synth cases, call the library through its
binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D

# Score tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| (1e-3 relative / 1e-2 absolute,
# read as numpy's allclose).
ATOL, RTOL = 1e-2, 1e-3


def have_gpu() -> bool:
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")
    if not D.library_path().exists():
        pytest.fail("libdsaidx.so is not built")


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t):
    return t.cpu().numpy()


class Uploaded:
    """A synth case with its arrays on the GPU."""

    def __init__(self, case):
        self.case = case
        kind = type(case).__name__
        self.kind = kind
        # prefill chunks (and cases that ask to be run as one) go through the prefill entry
        self.prefill = kind == "Dense" and (case.name == "prefill_chunk" or bool(case.meta.get("as_prefill")))
        self.q, self.w = dev(case.q), dev(case.w)
        if kind in ("Paged", "PagedSparse"):
            self.k, self.sc = dev(case.k_pages), dev(case.k_scale_pages)
            self.bt, self.sl = dev(case.block_table), dev(case.seq_lens)
            self.rr = dev(case.row_req)
            if kind == "PagedSparse":
                self.cand, self.nc = dev(case.cand), dev(case.n_cols)
        else:
            self.k, self.sc = dev(case.k), dev(case.k_scale)
            self.ks, self.ke = dev(case.row_ks), dev(case.row_ke)
        if kind == "Sparse":
            self.cand, self.nc = dev(case.cand), dev(case.n_cols)

    def logits(self, ld=None):
        c = self.case
        if self.kind == "Dense":
            return D.idx_logits(self.q, self.w, self.k, self.sc, self.ks, self.ke, k_dtype=c.k_dtype,
                                ld=ld or c.max_cols, prefill=self.prefill)
        if self.kind == "Paged":
            return D.idx_logits_paged(self.q, self.w, self.k, self.sc, self.bt, self.sl,
                                      k_dtype=c.k_dtype, row_req=self.rr, ld=ld)
        if self.kind == "PagedSparse":
            return D.idx_logits_paged_sparse_blocks(self.q, self.w, self.k, self.sc, self.bt, self.sl, self.cand,
                                                    self.nc, k_dtype=c.k_dtype, block_size=c.block,
                                                    row_req=self.rr, ld=ld)
        return D.idx_logits_sparse_blocks(self.q, self.w, self.k, self.sc, self.ks, self.ke,
                                          self.cand, self.nc, k_dtype=c.k_dtype,
                                          block_size=c.block, ld=ld)

    def problem(self):
        c = self.case
        if self.kind == "Dense":
            return D.dense_problem(self.q, self.w, self.k, self.sc, self.ks, self.ke,
                                   k_dtype=c.k_dtype, max_cols=c.max_cols, prefill=self.prefill)
        if self.kind == "Paged":
            return D.paged_problem(self.q, self.w, self.k, self.sc, self.bt, self.sl,
                                   k_dtype=c.k_dtype, row_req=self.rr)
        if self.kind == "PagedSparse":
            return D.paged_sparse_problem(self.q, self.w, self.k, self.sc, self.bt, self.sl, self.cand, self.nc,
                                          k_dtype=c.k_dtype, block_size=c.block, row_req=self.rr)
        return D.sparse_problem(self.q, self.w, self.k, self.sc, self.ks, self.ke, self.cand,
                                self.nc, k_dtype=c.k_dtype, block_size=c.block)

    def select(self, k=None, sorted=True):
        k = self.case.topk if k is None else k
        return D.idx_select(self.problem(), k, sorted=sorted)


# (check, workload, detail) -> (max |err|, max err/tol, rows checked): printed as a parity
# summary at the end of the run (tests/conftest.py)
PARITY = {}


def record(check: str, workload: str, detail: str, max_err: float, max_ratio: float, rows: str) -> None:
    PARITY[(check, workload, detail)] = (max_err, max_ratio, rows)


def score_error_stats(gpu, ref):
    """(max |gpu - ref|, max |gpu - ref| / tol) over the finite reference scores."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    ri = np.isneginf(ref)
    g, r = gpu[~ri].astype(np.float64), ref[~ri].astype(np.float64)
    if not g.size:
        return 0.0, 0.0
    err = np.abs(g - r)
    return float(err.max()), float((err / (ATOL + RTOL * np.abs(r))).max())


def assert_scores_close(gpu, ref, what=""):
    """Same set of unscored (-inf) positions, finite scores within the tolerance."""
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} != {ref.shape}"
    gi, ri = np.isneginf(gpu), np.isneginf(ref)
    bad = np.argwhere(gi != ri)
    assert bad.size == 0, f"{what}: -inf mask differs at {bad[:5].tolist()}"
    assert not np.isnan(gpu).any(), f"{what}: NaN in GPU scores"
    g, r = gpu[~ri].astype(np.float64), ref[~ri].astype(np.float64)
    err = np.abs(g - r)
    lim = ATOL + RTOL * np.abs(r)
    worst = int(np.argmax(err - lim)) if err.size else 0
    assert np.all(err <= lim), (f"{what}: {int((err > lim).sum())} scores outside tolerance; "
                                f"worst |d|={err[worst]:.3g} at ref={r[worst]:.6g}")
    return float(err.max()) if err.size else 0.0


def assert_selection_matches(gpu_idx, ref_idx, ref_scores_of, kth_ref, what=""):
    """End-to-end rule: overall overlap >= 0.999 and every index in the symmetric difference
    scores within twice the tolerance of the oracle's k-th value.
    ``ref_scores_of(r, idx_array)`` returns the oracle scores of the given positions."""
    total, inter = 0, 0
    worst = 0.0  # largest |score - k-th| / limit over the disagreements
    for r in range(ref_idx.shape[0]):
        a = set(int(x) for x in gpu_idx[r] if x >= 0)
        b = set(int(x) for x in ref_idx[r] if x >= 0)
        assert len(a) == len(b), f"{what}: row {r} selects {len(a)} != {len(b)}"
        total += len(b)
        inter += len(a & b)
        diff = np.array(sorted(a ^ b), dtype=np.int64)
        if diff.size:
            v = ref_scores_of(r, diff).astype(np.float64)
            kth = float(kth_ref[r])
            lim = 2 * (ATOL + RTOL * abs(kth))
            worst = max(worst, float((np.abs(v - kth) / lim).max()))
            assert np.all(np.abs(v - kth) <= lim), (
                f"{what}: row {r}: disagreement far from the cut (k-th {kth}, got {v[:5]})")
    assert total == 0 or inter / total >= 0.999, f"{what}: overlap {inter}/{total}"
    assert_selection_matches.worst = worst
    return inter, total
