"""GPU: idx_select_noalloc (idx_select on the library's static device scratch) against
idx_select with a workspace, through the C ABI: the same indices and values bit for bit on
two calls in a row, the second with a smaller problem, on the one-pass path (paged decode
at the 64-row x 128K workload shape, then fewer and shorter rows) and on the scores-then-
top-k path (a prefill chunk, then a smaller one); a problem larger than the scratch is
refused before anything runs; the calls leave torch's allocator untouched."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import synth
from gpu_util import Uploaded, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _both(up, k, sorted=True):
    """(idx, val) from idx_select with a workspace, then from idx_select_noalloc."""
    p = up.problem()
    r_idx, r_val = D.idx_select(p, k, sorted=sorted)
    torch.cuda.synchronize()
    rows = up.case.rows
    out_idx = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    out_val = torch.full((rows, k), 7.0, dtype=torch.float32, device="cuda")
    before = torch.cuda.memory_allocated()
    D.idx_select_noalloc(p, k, sorted=sorted, out_idx=out_idx, out_val=out_val)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return (host(r_idx), host(r_val)), (host(out_idx), host(out_val))


def _same(name, ref, got, sorted=True):
    (ri, rv), (gi, gv) = ref, got
    if sorted:
        assert np.array_equal(gi, ri), f"{name}: indices differ"
        assert np.array_equal(gv, rv), f"{name}: values differ"
    else:
        for r in range(ri.shape[0]):
            assert sorted_row(gi[r]) == sorted_row(ri[r]), f"{name}: row {r} differs as a set"


def sorted_row(a):
    return sorted(a.tolist())


def test_one_pass_large_then_small():
    require_gpu()
    big = synth.paged_decode(poison=False)  # 64 rows, 64K..128K keys, k = 2048
    need = D.idx_select_workspace(Uploaded(big).problem(), 2048)
    say(f"[no-alloc] paged 64 x 128K: workspace {need} bytes of {D.IDX_NOALLOC_SCRATCH_BYTES}")
    assert need <= D.IDX_NOALLOC_SCRATCH_BYTES
    up = Uploaded(big)
    _same("paged 64x128K", *_both(up, 2048))
    small = synth.paged_decode(seed=301, rows=12, min_len=500, max_len=20000)
    up = Uploaded(small)
    say("[no-alloc] paged 12 rows, up to 20K keys")
    _same("paged 12 rows", *_both(up, 2048))
    _same("paged 12 rows k=300 unsorted", *_both(up, 300, sorted=False), sorted=False)


def test_two_pass_large_then_small():
    require_gpu()
    for seed, q_tokens, prior, k in ((302, 512, 3000, 2048), (303, 260, 100, 512)):
        say(f"[no-alloc] prefill chunk {q_tokens} tokens after {prior}, k={k}")
        up = Uploaded(synth.prefill_chunk(seed=seed, q_tokens=q_tokens, prior=prior))
        _same(f"prefill {q_tokens}", *_both(up, k))


def test_too_large_is_refused():
    """A dense problem whose declared width needs more workspace than the scratch holds
    (the key arrays stay small: the call must be refused before anything runs)."""
    require_gpu()
    case = synth.batched_decode(seed=304, rows=16, n=1000)
    up = Uploaded(case)
    p = D.dense_problem(up.q, up.w, up.k, up.sc, up.ks, up.ke, k_dtype=case.k_dtype, max_cols=1 << 24)
    assert D.idx_select_workspace(p, 2048) > D.IDX_NOALLOC_SCRATCH_BYTES
    out_idx = torch.full((case.rows, 2048), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(D.IdxError) as e:
        D.idx_select_noalloc(p, 2048, out_idx=out_idx)
    assert e.value.status == D.IDX_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int((out_idx != -7).sum()) == 0, "nothing may run"
