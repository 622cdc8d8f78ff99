"""GPU idx_topk against the oracle's top-k, bit for bit: on oracle scores of the small
workloads, on adversarial rows (ties, few levels, sorted runs, signed zeros, absent
entries, short rows), and on rows of the full-size shapes."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import oracle as O
import synth
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _check(lg, k, lens=None, what=""):
    g_idx, g_val = D.idx_topk(dev(lg), k, lens=dev(lens))
    r_idx, r_val = O.topk(lg, k, lens)
    g_idx, g_val = host(g_idx), host(g_val)
    bad = np.argwhere(g_idx != r_idx)
    assert bad.size == 0, f"{what}: first mismatch at {bad[:3].tolist()}"
    assert np.array_equal(g_val, r_val), f"{what}: values differ"


def adversarial_rows(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = [
        rng.standard_normal(n),                                  # distinct
        np.full(n, 2.5),                                         # all equal
        rng.integers(0, 4, n) * 1.0,                             # four levels
        np.arange(n, dtype=np.float64),                          # ascending
        -np.arange(n, dtype=np.float64),                         # descending
        np.where(rng.random(n) < 0.5, 0.0, -0.0),                # signed zeros only
        np.linspace(0.0, 1.0, n) ** 3,                           # recency-like ramp
        np.where(rng.random(n) < 0.9, -np.inf, rng.standard_normal(n)),   # mostly absent
        np.where(rng.random(n) < 0.01, np.nan, rng.integers(-3, 3, n) * 0.5),  # NaN holes, ties
        rng.standard_normal(n) * 1e-30,                          # tiny magnitudes
        np.where(rng.random(n) < 0.5, 3.0e38, -3.0e38),          # huge magnitudes
        np.full(n, -np.inf),                                     # nothing to select
    ]
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("k", [1, 7, 256, 512, 1024, 2048])
def test_adversarial_rows(k):
    require_gpu()
    # widths up to 16384 take the one-kernel path; wider rows the histogram / filter /
    # finish path, whose candidate list overflows (falling back to a full-row select) on
    # the all-equal and few-level rows
    for n in (5, 2047, 2048, 2049, 9000, 16384, 16385, 40000):
        lg = adversarial_rows(n, seed=n + k)
        _check(lg, k, what=f"adversarial n={n} k={k}")
        lens = np.random.default_rng(n).integers(0, n + 1, lg.shape[0]).astype(np.int32)
        _check(lg, k, lens=lens, what=f"adversarial+lens n={n} k={k}")


@pytest.mark.parametrize("k", [7, 2048])
def test_adversarial_rows_many(k):
    """More rows than compute units (512 threads per row on the one-pass bucket path): the
    adversarial rows repeated, plus rows whose buckets cannot order them (one outlier
    squeezes the rest into a few buckets, a cluster of near-equal scores at the cut), each
    row against the oracle, sorted and unsorted."""
    require_gpu()
    for n in (5, 2049, 8192):
        base = adversarial_rows(n, seed=3 * n + k)
        rng = np.random.default_rng(n + k)
        outlier = rng.standard_normal(n).astype(np.float32)
        outlier[n // 3] = 1e30
        cluster = rng.standard_normal(n).astype(np.float32)
        cluster[: n // 2] = np.float32(1.0) + rng.integers(0, 3, n // 2).astype(np.float32) * np.float32(2 ** -20)
        lg = np.concatenate([np.tile(base, (26, 1)), outlier[None], cluster[None]])
        lens = rng.integers(0, n + 1, lg.shape[0]).astype(np.int32)
        _check(lg, k, what=f"many rows n={n} k={k}")
        _check(lg, k, lens=lens, what=f"many rows+lens n={n} k={k}")
        r_idx, _ = O.topk(lg, k)
        g_idx, _ = D.idx_topk(dev(lg), k, sorted=False)
        g_idx = host(g_idx)
        for r in range(lg.shape[0]):
            assert sorted(g_idx[r].tolist()) == sorted(r_idx[r].tolist()), f"unsorted n={n} k={k} row {r}"


SMALL = {
    "tiny_dense": lambda: synth.tiny_dense(),
    "dense_fp8": lambda: synth.batched_decode(seed=121, rows=4, n=5000, ragged=True),
    "paged_fp8": lambda: synth.paged_decode(seed=122, rows=4, min_len=1000, max_len=6000),
    "sparse_mxfp4": lambda: synth.sparse_blocks(seed=123, rows=4, ctx=8192, n_blocks=20, ragged=True),
    "prefill": lambda: synth.prefill_chunk(seed=124, q_tokens=64, prior=2000),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_on_oracle_scores(name):
    require_gpu()
    case = SMALL[name]()
    _, _, lg = O.select_case(case, with_logits=True)
    for k in sorted({min(case.topk, 2048), 256, 1024, 2048}):
        _check(lg, k, what=f"{name} k={k}")


def test_unsorted_flag_gives_the_same_set():
    require_gpu()
    lg = adversarial_rows(3000, seed=5)
    r_idx, _ = O.topk(lg, 700)
    g_idx, _ = D.idx_topk(dev(lg), 700, sorted=False)
    g_idx = host(g_idx)
    for r in range(lg.shape[0]):
        assert sorted(g_idx[r].tolist()) == sorted(r_idx[r].tolist()), f"row {r}"


@pytest.mark.parametrize("shape", [(64, 131072, 2048), (64, 131072, 512), (32, 32768, 2048),
                                   (4096, 8192, 2048), (64, 8192, 2048),
                                   # one or few very long rows: the most segments per row
                                   (1, 1 << 22, 2048), (3, 1 << 20, 1024)])
def test_full_size_shapes(shape):
    """Rows of the workloads' sizes (synthetic scores with heavy ties), every row checked."""
    require_gpu()
    rows, n, k = shape
    rng = np.random.default_rng(rows + n + k)
    lg = (rng.integers(-2000, 2000, size=(rows, n)) / 64).astype(np.float32)
    lens = rng.integers(n // 2, n + 1, rows).astype(np.int32)
    say(f"[topk] full shape rows={rows} n={n} k={k}")
    _check(lg, k, lens=lens, what=f"shape {shape}")
