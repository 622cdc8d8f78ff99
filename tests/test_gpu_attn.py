"""GPU idx_sparse_attn_paged against the oracle: attention over each row's selected
entries of a paged 576-element cache (out = softmax(scale * q . c) . c[:512], and the
log-sum-exp), for every head count, selections of 1 .. 2048 positions with padding,
out-of-range and duplicate positions, permuted page tables and a row -> request map,
peaked and flat score distributions, rows without any valid entry, and under graph
replay.

Tolerance: scores and the softmax run in fp32 on bf16 inputs (products exact), and the
weights are rounded to bf16 for the value product, so each output element is off by at
most about 2^-9 of the largest selected |value| plus fp32 rounding; the test allows
2^-8 of it. lse: 1e-4 absolute."""
import numpy as np
import pytest
import torch

import dsa_lightning_indexer_idx_amd as D
import oracle as O
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


def bf16_bits(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_case(seed, rows, heads, lens, k, q_std=1.0, pad=0.0, dup=False, permute=True, row_req=False):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    npg = (lens + 63) // 64
    P = int(npg.sum()) + 3
    kv = bf16_bits(rng.standard_normal((P, 64, 576)))
    q = bf16_bits(rng.standard_normal((rows, heads, 576)) * q_std / np.sqrt(576))
    perm = rng.permutation(P).astype(np.int32) if permute else np.arange(P, dtype=np.int32)
    bt_ld = int(npg.max())
    reqs = rng.permutation(rows).astype(np.int32) if row_req else np.arange(rows, dtype=np.int32)
    bt = np.full((rows, bt_ld), -1, np.int32)
    off = 0
    for i in range(rows):
        bt[reqs[i], :npg[i]] = perm[off:off + npg[i]]
        off += int(npg[i])
    idx = np.full((rows, k), -1, np.int32)
    for i in range(rows):
        n = min(k, int(lens[i])) if not dup else k
        sel = rng.choice(int(lens[i]), size=n, replace=dup)
        idx[i, :n] = sel
        if pad:
            drop = rng.random(k) < pad
            idx[i, drop] = rng.choice([-1, int(lens[i]), int(lens[i]) + 77], size=int(drop.sum()))
    return dict(q=q, kv=kv, bt=bt, sl=lens, idx=idx, req=reqs if row_req else None)


def check(case, scale, what):
    c = case
    rows, heads, _ = c["q"].shape
    k = c["idx"].shape[1]
    say(f"sparse attn: {what} rows={rows} heads={heads} k={k}")
    g_out, g_lse = D.idx_sparse_attn_paged(dev(c["q"]), dev(c["kv"]), dev(c["bt"]), dev(c["sl"]), dev(c["idx"]),
                                           scale, row_req=dev(c["req"]))
    torch.cuda.synchronize()
    r_out, r_lse = O.sparse_attn_paged(c["q"], c["kv"], c["bt"], c["sl"], c["idx"], scale, row_req=c["req"])
    g_out, g_lse = host(g_out), host(g_lse)
    vals = O._bf16_table()[c["kv"]]
    for r in range(rows):
        req = r if c["req"] is None else int(c["req"][r])
        sel = [int(s) for s in c["idx"][r] if 0 <= s < c["sl"][r]]
        if not sel:
            assert np.all(g_out[r] == 0) and np.all(g_lse[r] == -np.inf), f"{what}: empty row {r}"
            continue
        vmax = max(np.abs(vals[c["bt"][req][s // 64], s % 64, :512]).max() for s in sel)
        tol = 2.0 ** -8 * vmax + 1e-5
        err = np.abs(g_out[r] - r_out[r]).max()
        assert err <= tol, f"{what}: row {r} max error {err:.3g} > {tol:.3g}"
        assert np.allclose(g_lse[r], r_lse[r], rtol=0, atol=1e-4), f"{what}: row {r} lse"
    return g_out, g_lse


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_heads_and_sizes(heads):
    require_gpu()
    for seed, lens, k, q_std in ((80, [300, 1000, 77], 64, 1.0), (81, [5000, 2100], 2048, 4.0),
                                 (82, [40, 3000, 9000], 517, 0.2)):
        c = make_case(seed + heads, len(lens), heads, lens, k, q_std=q_std, pad=0.1)
        check(c, 1 / np.sqrt(192), f"heads {heads} seed {seed}")


def test_single_and_duplicate_positions():
    require_gpu()
    c = make_case(90, 3, 64, [500, 500, 500], 1)
    out, lse = check(c, 0.07, "one position")
    c = make_case(91, 2, 32, [100, 3000], 300, dup=True)
    check(c, 0.07, "duplicates")


def test_tables_and_empty_rows():
    require_gpu()
    c = make_case(92, 4, 128, [7000, 64, 1, 20000], 2048, q_std=2.0, pad=0.3, row_req=True)
    c["idx"][2, :] = -1          # no valid entry
    c["idx"][1, :] = 99999       # past the length
    check(c, 1 / np.sqrt(192), "row_req, empty rows")
    c = make_case(93, 2, 16, [4096, 4096], 2048, permute=False)
    check(c, 0.01, "identity table, flat scores")


@pytest.mark.parametrize("heads", [16, 64, 128])
def test_padding_ignores_nonfinite_cache_entries(heads):
    """Padded and out-of-range positions must not read what the cache holds: physical
    page 0 (flat entry 0) and the spare pages carry bf16 NaN and Inf, none of them is
    referenced by a valid position, and the rows carry -1 / past-length padding; the
    output is finite and matches the oracle."""
    require_gpu()
    c = make_case(95 + heads, 3, heads, [3000, 700, 130], 512, q_std=2.0, pad=0.4)
    bt = c["bt"]
    used = set(int(x) for x in bt.ravel() if x >= 0)
    spare = [pg for pg in range(c["kv"].shape[0]) if pg not in used]
    if 0 in used:  # move page 0's content to a spare page so that page 0 is unreferenced
        s0 = spare[0]
        c["kv"][s0] = c["kv"][0]
        bt[bt == 0] = s0
        spare = [pg for pg in range(c["kv"].shape[0]) if pg not in set(int(x) for x in bt.ravel() if x >= 0)]
    assert 0 in spare
    for pg in spare:
        c["kv"][pg, :, 0::2] = 0x7FC0  # NaN
        c["kv"][pg, :, 1::2] = 0x7F80  # +Inf
    out, lse = check(c, 1 / np.sqrt(192), f"nonfinite unreferenced entries, {heads} heads")
    assert np.all(np.isfinite(out)), "padding leaked a non-finite cache value"


@pytest.mark.parametrize("heads", [128, 16])
def test_graph_replay_matches_eager(heads):
    require_gpu()
    c = make_case(94, 8, heads, [6000] * 8, 1024, q_std=1.5, pad=0.05)
    q, kv, bt, sl, idx = dev(c["q"]), dev(c["kv"]), dev(c["bt"]), dev(c["sl"]), dev(c["idx"])
    out = torch.empty((8, heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((8, heads), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, D.idx_sparse_attn_workspace(8, heads, 1024)), dtype=torch.uint8, device="cuda")
    say(f"sparse attn: eager, {heads} heads")
    D.idx_sparse_attn_paged(q, kv, bt, sl, idx, 0.07, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    want_o, want_l = host(out).copy(), host(lse).copy()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        D.idx_sparse_attn_paged(q, kv, bt, sl, idx, 0.07, out=out, lse=lse, workspace=ws, stream=s)
        torch.cuda.synchronize()
        g.capture_begin()
        D.idx_sparse_attn_paged(q, kv, bt, sl, idx, 0.07, out=out, lse=lse, workspace=ws, stream=s)
        g.capture_end()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(7.0)
        ws.fill_(0x55)
        torch.cuda.synchronize()
        say(f"sparse attn: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), want_o) and np.array_equal(host(lse), want_l), f"replay {i}"


def test_full_size_long_decode():
    """The long paged decode's shape: 64 rows of U{65536..131072} positions in 64-token
    pages (the indexer workload's table), 2048 selected positions per row drawn at random;
    a 576-element bf16 cache of ~98K pages made on the GPU by torch's seeded generator.
    128 heads, then the first 16 of them (one GPU's share of 128 heads split 8 ways, its
    own single-wave kernel), each in the launch shape the bench times. Rows 0 and 63 are
    checked against the oracle (their pages copied back)."""
    import synth
    require_gpu()
    c = synth.paged_decode(poison=False)
    P = c.k_pages.shape[0]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    kv = torch.randn((P, 64, 576), generator=gen, device="cuda", dtype=torch.bfloat16)
    q128 = (torch.randn((64, 128, 576), generator=gen, device="cuda", dtype=torch.float32) / 16).to(torch.bfloat16)
    rng = np.random.default_rng(12)
    idx = np.stack([rng.choice(int(n), size=2048, replace=False) for n in c.seq_lens]).astype(np.int32)
    kvr = {}
    for r in (0, 63):
        npg = int((c.seq_lens[r] + 63) // 64)
        pages = torch.from_numpy(c.block_table[r, :npg].astype(np.int64)).cuda()
        kvr[r] = kv.index_select(0, pages).view(torch.int16).cpu().numpy().view(np.uint16)
    for heads in (128, 16):
        q = q128[:, :heads].contiguous()
        say(f"sparse attn: full size, {heads} heads")
        out, lse = D.idx_sparse_attn_paged(q, kv, dev(c.block_table), dev(c.seq_lens), dev(idx), 1 / np.sqrt(192))
        torch.cuda.synchronize()
        out, lse = host(out), host(lse)
        qb = q.view(torch.int16).cpu().numpy().view(np.uint16)
        for r in (0, 63):
            npg = kvr[r].shape[0]
            bt = np.arange(npg, dtype=np.int32)[None]
            r_out, r_lse = O.sparse_attn_paged(qb[r:r + 1], kvr[r], bt, c.seq_lens[r:r + 1], idx[r:r + 1],
                                               1 / np.sqrt(192))
            vmax = np.abs(O._bf16_table()[kvr[r][..., :512]]).max()
            err = np.abs(out[r] - r_out[0]).max()
            assert err <= 2.0 ** -8 * vmax + 1e-5, f"full size, {heads} heads, row {r}: max error {err:.3g}"
            assert np.allclose(lse[r], r_lse[0], rtol=0, atol=1e-4), f"full size, {heads} heads, row {r}: lse"
