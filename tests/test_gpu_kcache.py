"""GPU key-cache writer against the oracle's writer, byte for byte, and end to end: keys
written by the GPU into pages score exactly like the oracle-written pages."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import oracle as O
import synth
from gpu_util import dev, host, require_gpu, say, assert_scores_close

pytestmark = pytest.mark.gpu


def _keys(rng, n):
    x = (rng.standard_normal((n, 128)) * rng.uniform(1e-3, 1e3, (n, 1))).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2, :] = 0.0
    x[2, 9] = -7.5e-3
    x[3, 17] = 6.0e4
    x[4, :64] = np.float32(2.0 ** -130)               # subnormal magnitudes
    x[5] = np.float32(448.0) * (np.arange(128) - 64)  # many exact fp8 values
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6], np.float32)
    for i in range(6, 12):                            # e2m1 grid points and ties, group max 6
        row = rng.choice(grid, 128) * rng.choice([-1, 1], 128)
        row[::32] = 6.0
        x[i] = row * np.float32(2.0) ** rng.integers(-10, 10)
    return synth.to_bf16_bits(x)


@pytest.mark.parametrize("kd", ["fp8", "mxfp4"])
@pytest.mark.parametrize("n", [1, 2, 3, 200, 5001])
def test_writer_matches_oracle(kd, n):
    require_gpu()
    rng = np.random.default_rng(n + (0 if kd == "fp8" else 1))
    n_slots = n + 37
    keys = _keys(rng, max(n, 12))[:n]
    slots = rng.permutation(n_slots)[:n].astype(np.int64)
    if n > 3:
        slots[1] = -1
    row, srow = (128, 1) if kd == "fp8" else (64, 4)
    cache = np.full((n_slots, row), 0x5A, np.uint8)
    sc = np.full(n_slots, 1234.5, np.float32) if kd == "fp8" else np.full((n_slots, 4), 0x5A, np.uint8)
    g_cache, g_sc = dev(cache), dev(sc)
    say(f"[kcache] {kd} n={n}")
    D.idx_kcache_write(dev(keys).view(torch.bfloat16), dev(slots), g_cache, g_sc, kd)
    O.kcache_write(keys, slots, kd, cache, sc)
    assert np.array_equal(host(g_cache), cache), "codes differ"
    assert np.array_equal(host(g_sc).view(np.uint8), sc.view(np.uint8)), "scales differ"
    assert D.idx_device_errors() == 0


def test_out_of_range_slot_is_skipped_and_reported():
    require_gpu()
    keys = _keys(np.random.default_rng(5), 12)[:4]
    slots = np.array([0, 5, 7, 2], np.int64)
    cache = torch.full((6, 128), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(6, dtype=torch.float32, device="cuda")
    D.idx_device_errors()
    D.idx_kcache_write(dev(keys).view(torch.bfloat16), dev(slots), cache, sc, "fp8")
    assert D.idx_device_errors() & D.IDX_DEVERR_SLOT
    ref = np.full((6, 128), 0x5A, np.uint8)
    ref_sc = np.zeros(6, np.float32)
    assert O.kcache_write(keys, slots, "fp8", ref, ref_sc) == 1
    assert np.array_equal(host(cache), ref) and np.array_equal(host(sc), ref_sc)


@pytest.mark.parametrize("kd", ["fp8", "mxfp4"])
def test_written_pages_score_like_the_oracle(kd):
    """Write a paged cache with the GPU writer, score it with idx_logits_paged, and compare
    with the oracle's scores over the oracle-written cache (the same bytes)."""
    require_gpu()
    rng = np.random.default_rng(11 if kd == "fp8" else 12)
    rows, page, n_pages = 3, 64, 40
    lens = np.array([1500, 64, 900], np.int32)
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = np.full((rows, 24), -1, np.int32)
    slot_of = []
    used = 0
    for r in range(rows):
        np_r = (lens[r] + page - 1) // page
        bt[r, :np_r] = perm[used:used + np_r]
        used += np_r
        s = np.arange(lens[r])
        slot_of.append(bt[r, s // page].astype(np.int64) * page + s % page)
    slots = np.concatenate(slot_of)
    keys = synth.to_bf16_bits((rng.standard_normal((slots.size, 128)) * 0.3).astype(np.float32))
    row = 128 if kd == "fp8" else 64
    g_pages = torch.zeros((n_pages, page, row), dtype=torch.uint8, device="cuda")
    g_sc = (torch.zeros((n_pages, page), dtype=torch.float32, device="cuda") if kd == "fp8"
            else torch.zeros((n_pages, page, 4), dtype=torch.uint8, device="cuda"))
    D.idx_kcache_write(dev(keys).view(torch.bfloat16), dev(slots), g_pages, g_sc, kd)
    ref_pages = np.zeros((n_pages * page, row), np.uint8)
    ref_sc = np.zeros(n_pages * page, np.float32) if kd == "fp8" else np.zeros((n_pages * page, 4), np.uint8)
    O.kcache_write(keys, slots, kd, ref_pages, ref_sc)
    assert np.array_equal(host(g_pages).reshape(ref_pages.shape), ref_pages)
    q = synth.to_fp8_e4m3fn(rng.standard_normal((rows, 64, 128)).astype(np.float32))
    w = (rng.standard_normal((rows, 64)) / 8).astype(np.float32)
    lg = host(D.idx_logits_paged(dev(q), dev(w), g_pages, g_sc, dev(bt), dev(lens), k_dtype=kd))
    ref = O.logits_paged(q, "fp8", w, ref_pages.reshape(n_pages, page, row),
                         ref_sc.reshape((n_pages, page) if kd == "fp8" else (n_pages, page, 4)), kd, bt, lens,
                         None, ld=lg.shape[1])
    assert_scores_close(lg, ref, f"written {kd} pages")
