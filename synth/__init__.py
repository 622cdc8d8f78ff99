"""Seeded synthetic inputs for the DSA lightning indexer.

This module serves both sides of every parity test (the GPU library and the CPU
oracle) and the benchmark. It holds none of the indexer's arithmetic: only random
draws, torch's own casts to bf16 and to fp8 e4m3fn, and the OCP Microscaling (MX)
v1.0 encoding of a Gaussian into e2m1 codes with UE8M0 group-32 scales, which is
the input preparation an MXFP4 key cache would receive from its writer.

Shapes follow the indexer cache on the pages: one 128-element key per token shared
by all 64 indexer heads (DeepSeek-V3.2 architecture, Eq. (1); the llama.cpp issue
notes the extra 128-element k_s cache), 64-token pages addressed by a per-request
block table, and candidate blocks with a valid sparse-column count per row
(vLLM sparse_indexer page, SparseMQARowsMetadata).

Every array has its own child stream of ``SeedSequence(seed)`` so that a case is
reproducible array by array. Poison fill (fp8 code 0x7F = NaN, scale NaN, UE8M0
0xFF = NaN) marks bytes a correct kernel never reads or always masks.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

HEADS = 64
DIM = 128
FP8_NAN = 0x7F
UE8M0_NAN = 0xFF

_STREAMS = ("q", "w", "k", "scale", "lens", "table", "cand", "poison", "extra")


def _rngs(seed: int) -> dict[str, np.random.Generator]:
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(_STREAMS, kids)}


# ----------------------------------------------------------------------------- encodings


def to_fp8_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn byte codes (torch cast, RNE), clamped to +-448 first
    because torch's cast does not saturate."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (torch cast, RNE) as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_mxfp4(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode float rows [..., D] (D % 32 == 0) as MXFP4 following OCP MX v1.0:
    per group of 32 the shared exponent is floor(log2(amax)) - 2 (2 = emax of e2m1),
    stored biased by 127 as UE8M0; each element v / 2^X is rounded to nearest-even on
    the e2m1 grid and saturated at +-6. Returns (codes [..., D/2] uint8 with element 2j
    in the low nibble of byte j, scales [..., D/32] uint8).

    The e2m1 grid has step 0.5 below 2, step 1 in [2, 4) and step 2 in [4, 6], so the
    rounding is rint (round half to even) of the magnitude in units of the local step;
    a tie at a step boundary (1.75, 3.5) rounds to the even code either way."""
    x = np.asarray(x, dtype=np.float32)
    *lead, d = x.shape
    assert d % 32 == 0
    g = x.reshape(*lead, d // 32, 32)
    amax = np.abs(g).max(axis=-1)
    _, e = np.frexp(amax)  # amax = m 2^e with m in [0.5, 1): floor(log2(amax)) = e - 1
    xexp = np.where(amax > 0, e.astype(np.int32) - 1 - 2, -127)
    biased = np.clip(xexp + 127, 0, 254).astype(np.int32)
    scaled = np.ldexp(g, (127 - biased)[..., None]).astype(np.float32)  # exact: a power of two
    mag = np.minimum(np.abs(scaled), np.float32(6.0))
    code = np.where(mag < 2, np.rint(mag * 2),
                    np.where(mag < 4, np.rint(mag) + 2, np.rint(mag * 0.5) + 4)).astype(np.uint8)
    code |= np.where(scaled < 0, 8, 0).astype(np.uint8)
    code = code.reshape(*lead, d)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, biased.astype(np.uint8)


def _normal(rng, shape, scale=1.0, chunk=1 << 26) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        n = min(chunk, out.size - s)
        out[s:s + n] = rng.standard_normal(n, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


_CHUNK = 1 << 24


def _fp8_normal(rng, shape) -> np.ndarray:
    """N(0,1) draws cast to e4m3fn codes. Fixed 16M-element chunks each draw from their
    own stream seeded from ``rng`` and fill in parallel threads, so the result depends
    only on the seed, never on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    starts = list(range(0, n, _CHUNK))
    seeds = rng.integers(0, 2 ** 63, size=len(starts))

    def fill(i):
        s = starts[i]
        m = min(_CHUNK, n - s)
        g = np.random.Generator(np.random.PCG64(int(seeds[i])))
        out[s:s + m] = to_fp8_e4m3fn(g.standard_normal(m, dtype=np.float32))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


def _keys(rng, n: int, kdtype: str, scale_rng):
    """Key cache rows for n tokens: (codes, scales) in the layout of ``kdtype``."""
    if kdtype == "fp8":
        codes = _fp8_normal(rng, (n, DIM))
        scale = scale_rng.uniform(0.5, 2.0, size=n).astype(np.float32)
        return codes, scale
    if kdtype == "bf16":
        return to_bf16_bits(_normal(rng, (n, DIM), 1.0 / np.sqrt(DIM))), None
    if kdtype == "mxfp4":
        codes = np.empty((n, DIM // 2), np.uint8)
        scales = np.empty((n, DIM // 32), np.uint8)
        step = _CHUNK // DIM
        starts = list(range(0, n, step))
        seeds = rng.integers(0, 2 ** 63, size=len(starts))

        def fill(i):
            s = starts[i]
            m = min(step, n - s)
            g = np.random.Generator(np.random.PCG64(int(seeds[i])))
            codes[s:s + m], scales[s:s + m] = to_mxfp4(g.standard_normal((m, DIM), dtype=np.float32))

        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(starts))))
        return codes, scales
    raise ValueError(kdtype)


def _queries(rng, rows: int, qdtype: str) -> np.ndarray:
    if qdtype == "fp8":
        return _fp8_normal(rng, (rows, HEADS, DIM))
    if qdtype == "bf16":
        return to_bf16_bits(_normal(rng, (rows, HEADS, DIM), 1.0 / np.sqrt(DIM)))
    raise ValueError(qdtype)


def _weights(rng, rows: int) -> np.ndarray:
    return _normal(rng, (rows, HEADS), 1.0 / 8.0)


def _poison_keys(codes: np.ndarray, scale, kdtype: str, sel) -> None:
    """Overwrite token rows ``sel`` with NaN codes / NaN scales."""
    if kdtype == "fp8":
        codes[sel] = FP8_NAN
        scale[sel] = np.nan
    elif kdtype == "mxfp4":
        scale[sel] = UE8M0_NAN
    elif kdtype == "bf16":
        codes[sel] = 0x7FC0


# ----------------------------------------------------------------------------- cases


@dataclass
class Dense:
    """Rows scoring the contiguous key range [row_ks, row_ke) of one flat key array."""
    name: str
    q: np.ndarray
    q_dtype: str
    w: np.ndarray
    k: np.ndarray
    k_scale: np.ndarray | None
    k_dtype: str
    row_ks: np.ndarray
    row_ke: np.ndarray
    topk: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def max_cols(self) -> int:
        return int((self.row_ke - self.row_ks).max()) if self.rows else 0

    @property
    def tokens(self) -> int:
        return int((self.row_ke - self.row_ks).sum())


@dataclass
class Paged:
    """Rows whose logical token s lives in page block_table[req][s // page], slot s % page."""
    name: str
    q: np.ndarray
    q_dtype: str
    w: np.ndarray
    k_pages: np.ndarray          # fp8: [P, page, 128] u8; mxfp4: [P, page, 64] u8
    k_scale_pages: np.ndarray    # fp8: [P, page] f32;     mxfp4: [P, page, 4] u8
    k_dtype: str
    page_size: int
    block_table: np.ndarray      # [n_req, bt_ld] int32
    seq_lens: np.ndarray         # [rows] int32
    row_req: np.ndarray | None   # [rows] int32 or None (identity)
    topk: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def max_cols(self) -> int:
        return int(self.block_table.shape[1] * self.page_size)

    @property
    def tokens(self) -> int:
        return int(self.seq_lens.sum())


@dataclass
class Sparse:
    """Two-level rows: score only the candidate blocks cand[r][:] of the row's key range.
    Column c maps to token cand[r][c // block] * block + c % block (relative to row_ks)."""
    name: str
    q: np.ndarray
    q_dtype: str
    w: np.ndarray
    k: np.ndarray
    k_scale: np.ndarray | None
    k_dtype: str
    row_ks: np.ndarray
    row_ke: np.ndarray
    cand: np.ndarray             # [rows, cand_ld] int32, sorted unique block ids
    n_cols: np.ndarray           # [rows] int32 valid sparse columns ("end")
    block: int
    topk: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def max_cols(self) -> int:
        return int(self.cand.shape[1] * self.block)

    @property
    def tokens(self) -> int:
        return int(self.n_cols.sum())


def tiny_dense(seed: int = 1, n: int = 4096, rows: int = 1, topk: int = 256) -> Dense:
    """One decode row over n bf16 keys; q, K ~ N(0,1)/sqrt(128), w ~ N(0,1)/8."""
    r = _rngs(seed)
    q = _queries(r["q"], rows, "bf16")
    w = _weights(r["w"], rows)
    k, _ = _keys(r["k"], rows * n, "bf16", r["scale"])
    ks = (np.arange(rows) * n).astype(np.int32)
    return Dense("tiny_dense", q, "bf16", w, k, None, "bf16", ks, ks + np.int32(n), topk,
                 {"n": n})


def batched_decode(seed: int = 2, rows: int = 32, n: int = 32768, topk: int = 2048,
                   kdtype: str = "fp8", ragged: bool = False, gap: int = 0) -> Dense:
    """Rows each with its own contiguous context of n tokens in one flat key array,
    row r at [r*(n+gap), r*(n+gap)+len_r). ``ragged`` draws len_r ~ U{1..n};
    gap tokens between rows are poisoned."""
    r = _rngs(seed)
    qd = "bf16" if kdtype == "bf16" else "fp8"
    q = _queries(r["q"], rows, qd)
    w = _weights(r["w"], rows)
    stride = n + gap
    k, sc = _keys(r["k"], rows * stride, kdtype, r["scale"])
    lens = (r["lens"].integers(1, n + 1, size=rows) if ragged else np.full(rows, n)).astype(np.int32)
    ks = (np.arange(rows) * stride).astype(np.int32)
    ke = (ks + lens).astype(np.int32)
    for i in range(rows):
        _poison_keys(k, sc, kdtype, slice(int(ke[i]), int(ks[i]) + stride))
    return Dense("batched_decode", q, qd, w, k, sc, kdtype, ks, ke, topk,
                 {"n": n, "ragged": ragged, "gap": gap})


def prefill_chunk(seed: int = 4, q_tokens: int = 4096, prior: int = 4096, topk: int = 2048,
                  kdtype: str = "fp8") -> Dense:
    """A prefill chunk: query i sits at position prior+i and sees keys [0, prior+i]
    inclusive (causal, self included), so row_ks = 0 and row_ke = prior+i+1."""
    r = _rngs(seed)
    q = _queries(r["q"], q_tokens, "fp8")
    w = _weights(r["w"], q_tokens)
    k, sc = _keys(r["k"], prior + q_tokens, kdtype, r["scale"])
    ks = np.zeros(q_tokens, np.int32)
    ke = (prior + 1 + np.arange(q_tokens)).astype(np.int32)
    return Dense("prefill_chunk", q, "fp8", w, k, sc, kdtype, ks, ke, topk,
                 {"q_tokens": q_tokens, "prior": prior})


def paged_decode(seed: int = 3, rows: int = 64, min_len: int = 65536, max_len: int = 131072,
                 page: int = 64, topk: int = 2048, kdtype: str = "fp8", poison: bool = True,
                 spare_pages: int = 8, row_req: bool = False) -> Paged:
    """Long-context paged decode: len_r ~ U{min_len..max_len}; the physical page pool is
    a random permutation handed out in row order; the table is [n_req, max_len/page]
    with unused entries -1. Slots past len_r in the last page and ``spare_pages``
    unreferenced pages are poisoned. ``row_req`` maps rows to a shuffled request order."""
    r = _rngs(seed)
    q = _queries(r["q"], rows, "fp8")
    w = _weights(r["w"], rows)
    lens = r["lens"].integers(min_len, max_len + 1, size=rows).astype(np.int32)
    npg = (lens + page - 1) // page
    P = int(npg.sum()) + spare_pages
    codes, sc = _keys(r["k"], P * page, kdtype, r["scale"])
    perm = r["table"].permutation(P).astype(np.int32)
    bt_ld = (max_len + page - 1) // page
    reqs = r["table"].permutation(rows).astype(np.int32) if row_req else np.arange(rows, dtype=np.int32)
    bt = np.full((rows, bt_ld), -1, np.int32)
    off = 0
    for i in range(rows):
        bt[reqs[i], :npg[i]] = perm[off:off + npg[i]]
        off += int(npg[i])
    if poison:
        flat_sel = []
        for i in range(rows):
            last = int(bt[reqs[i], npg[i] - 1])
            used = int(lens[i] - (npg[i] - 1) * page)
            flat_sel.append(np.arange(last * page + used, (last + 1) * page))
        for p in perm[off:]:
            flat_sel.append(np.arange(int(p) * page, (int(p) + 1) * page))
        if flat_sel:
            _poison_keys(codes, sc, kdtype, np.concatenate(flat_sel))
    if kdtype == "fp8":
        kp, sp = codes.reshape(P, page, DIM), sc.reshape(P, page)
    else:
        kp, sp = codes.reshape(P, page, DIM // 2), sc.reshape(P, page, DIM // 32)
    return Paged("paged_decode", q, "fp8", w, kp, sp, kdtype, page, bt, lens,
                 reqs if row_req else None, topk,
                 {"min_len": min_len, "max_len": max_len, "pages": P})


def sparse_blocks(seed: int = 5, rows: int = 64, ctx: int = 131072, n_blocks: int = 64,
                  block: int = 128, topk: int = 2048, kdtype: str = "mxfp4",
                  ragged: bool = False, poison_noncand: bool = True) -> Sparse:
    """Two-level candidate-block rows: each row owns a contiguous context of ``ctx``
    tokens; ``n_blocks`` unique sorted candidate blocks of ``block`` tokens are drawn
    uniformly from the row's blocks. ``ragged`` shortens the row's valid length (so the
    last candidate block can be partly invalid) and the valid column count.
    ``poison_noncand`` fills tokens outside every candidate block with NaN scales
    instead of drawing them (they are never read)."""
    r = _rngs(seed)
    q = _queries(r["q"], rows, "fp8")
    w = _weights(r["w"], rows)
    nblk_row = (ctx + block - 1) // block
    assert n_blocks <= nblk_row
    if ragged:
        lens = r["lens"].integers(max(1, ctx // 2), ctx + 1, size=rows).astype(np.int32)
    else:
        lens = np.full(rows, ctx, np.int32)
    cand = np.empty((rows, n_blocks), np.int32)
    for i in range(rows):
        cand[i] = np.sort(r["cand"].choice(nblk_row, size=n_blocks, replace=False))
    if ragged:
        n_cols = r["cand"].integers(1, n_blocks * block + 1, size=rows).astype(np.int32)
    else:
        n_cols = np.full(rows, n_blocks * block, np.int32)
    n_keys = rows * ctx
    if poison_noncand:
        if kdtype == "fp8":
            codes = np.full((n_keys, DIM), FP8_NAN, np.uint8)
            sc = np.full(n_keys, np.nan, np.float32)
        else:
            codes = np.zeros((n_keys, DIM // 2), np.uint8)
            sc = np.full((n_keys, DIM // 32), UE8M0_NAN, np.uint8)
        toks = (np.arange(rows)[:, None, None] * ctx + cand[:, :, None] * block
                + np.arange(block)[None, None, :]).reshape(-1)
        toks = toks[toks < np.repeat(np.arange(rows) * ctx + ctx, n_blocks * block)]
        c2, s2 = _keys(r["k"], toks.size, kdtype, r["scale"])
        codes[toks] = c2
        sc[toks] = s2
    else:
        codes, sc = _keys(r["k"], n_keys, kdtype, r["scale"])
    ks = (np.arange(rows) * ctx).astype(np.int32)
    ke = (ks + lens).astype(np.int32)
    return Sparse("sparse_blocks", q, "fp8", w, codes, sc, kdtype, ks, ke, cand, n_cols,
                  block, topk, {"ctx": ctx, "n_blocks": n_blocks})


@dataclass
class PagedSparse:
    """Two-level rows over a paged cache: column c names the row's logical token
    cand[r][c // block] * block + c % block, which lives in page
    block_table[req][token // page], slot token % page (req = row_req[r] or r)."""
    name: str
    q: np.ndarray
    q_dtype: str
    w: np.ndarray
    k_pages: np.ndarray
    k_scale_pages: np.ndarray
    k_dtype: str
    page_size: int
    block_table: np.ndarray
    seq_lens: np.ndarray
    row_req: np.ndarray | None
    cand: np.ndarray
    n_cols: np.ndarray
    block: int
    topk: int
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def max_cols(self) -> int:
        return int(self.cand.shape[1] * self.block)

    @property
    def tokens(self) -> int:
        return int(self.n_cols.sum())


def page_sparse(sp: Sparse, page: int = 64, seed: int = 0, permute: bool = True, row_req: bool = False,
                spare_pages: int = 8) -> PagedSparse:
    """The candidate-block case ``sp`` with each row's context moved into pages: row r's
    tokens [row_ks, row_ks + ctx) fill its ctx / page pages, taken from a pool that is a
    random permutation (``permute``) with ``spare_pages`` poisoned pages besides; the table
    maps logical page p of request req(r) to its physical page; ``row_req`` shuffles the
    rows' requests. The page must be a multiple of the kernel's sparse block: candidate
    blocks longer than a page are handed over split into page-sized sparse blocks (each
    candidate block b becomes blocks b*f .. b*f + f - 1, f = block / page), which name the
    same tokens column for column. The scores of every column equal those of ``sp`` (same
    key bytes)."""
    g = np.random.default_rng([seed, 77])
    ctx = int(sp.meta["ctx"])
    assert ctx % page == 0 and page % 64 == 0
    if page % sp.block:
        assert sp.block % page == 0
        f = sp.block // page
        cand = (sp.cand.astype(np.int64)[:, :, None] * f + np.arange(f)[None, None, :]).reshape(sp.rows, -1)
        cand, block = cand.astype(np.int32), page
    else:
        cand, block = sp.cand, sp.block
    rows, npg = sp.rows, ctx // page
    P = rows * npg + spare_pages
    phys = (g.permutation(P) if permute else np.arange(P)).astype(np.int32)
    kb = sp.k.shape[1]
    if sp.k_dtype == "fp8":
        kp = np.full((P, page, kb), FP8_NAN, np.uint8)
        scp = np.full((P, page), np.nan, np.float32)
    else:
        kp = np.zeros((P, page, kb), np.uint8)
        scp = np.full((P, page) + sp.k_scale.shape[1:], UE8M0_NAN, np.uint8)
    used = phys[:rows * npg]
    kp[used] = sp.k[:rows * ctx].reshape(rows * npg, page, kb)
    scp[used] = sp.k_scale[:rows * ctx].reshape((rows * npg, page) + sp.k_scale.shape[1:])
    reqs = (g.permutation(rows) if row_req else np.arange(rows)).astype(np.int32)
    bt = np.full((rows, npg), -1, np.int32)
    for i in range(rows):
        bt[reqs[i]] = used[i * npg:(i + 1) * npg]
    lens = (sp.row_ke - sp.row_ks).astype(np.int32)
    return PagedSparse("paged_sparse_blocks", sp.q, sp.q_dtype, sp.w, kp, scp, sp.k_dtype, page, bt, lens,
                       reqs if row_req else None, cand, sp.n_cols, block, sp.topk,
                       {**sp.meta, "page": page, "permute": permute, "candidate_block": sp.block})


def paged_sparse_blocks(seed: int = 5, rows: int = 64, ctx: int = 131072, n_blocks: int = 64, block: int = 128,
                        page: int = 64, topk: int = 2048, kdtype: str = "mxfp4", ragged: bool = False,
                        row_req: bool = False, poison_noncand: bool = True) -> PagedSparse:
    """The two-level workload over a paged cache: sparse_blocks(...) paged with 64-token
    pages from a permuted pool (128-token candidate blocks handed over as pairs of 64-token
    sparse blocks)."""
    sp = sparse_blocks(seed=seed, rows=rows, ctx=ctx, n_blocks=n_blocks, block=block, topk=topk, kdtype=kdtype,
                       ragged=ragged, poison_noncand=poison_noncand)
    return page_sparse(sp, page=page, seed=seed, row_req=row_req)


@dataclass
class Scores:
    """A candidate-source layer's score matrix (fp32 [rows, ld]) with row lengths."""
    name: str
    logits: np.ndarray
    lens: np.ndarray
    block: int
    n_top: int
    info: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.logits.shape[0]


POISON_SCORE = np.float32(1e30)  # past a row's length: would win every block if read


def candidate_scores(seed: int = 7, rows: int = 64, min_len: int = 65536, max_len: int = 131072,
                     ld: int | None = None, block: int = 128, n_top: int = 64,
                     adversarial: bool = False) -> Scores:
    """Scores of a layer that scored its whole context, the input of the candidate-block
    step: len_r ~ U{min_len..max_len} (the long paged decode recipe), scores N(0, 1) in
    fp32, columns at or past len_r set to a huge poison score. ``adversarial`` gives row r
    the pattern r % 8 instead: Gaussian; multiples of 1/4 in [-3, 3) (many equal block
    maxima); one constant; signed zeros; Gaussian with -inf stretches (masked keys) and
    NaN holes; a row of fewer than n_top blocks; an empty row; huge magnitudes."""
    r = _rngs(seed)
    ld = max_len if ld is None else ld
    lens = r["lens"].integers(min_len, max_len + 1, size=rows).astype(np.int32)
    g = r["extra"]
    lg = g.standard_normal((rows, ld), dtype=np.float32)
    if adversarial:
        for i in range(rows):
            kind = i % 8
            if kind == 1:
                lg[i] = g.integers(-12, 12, ld) / 4
            elif kind == 2:
                lg[i] = 0.75
            elif kind == 3:
                lg[i] = np.where(g.random(ld) < 0.5, 0.0, -0.0)
            elif kind == 4:
                starts = g.integers(0, ld, 6)
                for s0 in starts:
                    lg[i, s0:s0 + int(g.integers(1, 4 * block))] = -np.inf
                lg[i, g.random(ld) < 0.01] = np.nan
            elif kind == 5:
                lens[i] = min(lens[i], max(1, (n_top // 2) * block - int(g.integers(0, block))))
            elif kind == 6:
                lens[i] = 0
            elif kind == 7:
                lg[i] = np.where(g.random(ld) < 0.5, 3.0e38, -3.0e38)
    for i in range(rows):
        lg[i, lens[i]:] = POISON_SCORE
    return Scores("candidate_scores", lg, lens, block, n_top,
                  {"min_len": min_len, "max_len": max_len, "adversarial": adversarial})


def paged_decode_mxfp4(seed: int = 6):
    """The long paged decode workload with MXFP4 keys (e2m1 codes + UE8M0 group scales)."""
    return paged_decode(seed=seed, kdtype="mxfp4")


def full_size(idx: int):
    """The five workloads at their stated sizes, by number 1..5; 6: workload 3 with MXFP4
    keys; 7: workload 5 over a paged cache (64-token pages, permuted pool)."""
    return {1: tiny_dense, 2: batched_decode, 3: paged_decode, 4: prefill_chunk,
            5: sparse_blocks, 6: paged_decode_mxfp4, 7: paged_sparse_blocks}[idx]()
