"""CPU oracle for the DSA lightning indexer (logits by Eq. (1), exact top-k).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users. The GPU library never imports, links or calls
anything here, and this package imports nothing from the GPU library.

The arithmetic lives in ``ref.c`` (plain C, fp64, one RNE rounding to fp32 per
logit); this module builds it with gcc and marshals numpy arrays. The few steps
written here in numpy are column bookkeeping, each citing the passage it follows.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "ref.c"
_LIB = _HERE / "libdsaidx_oracle.so"
DTYPES = {"bf16": 1, "fp8": 2, "mxfp4": 3}
HEADS = 64
DIM = 128

_lib = None


def build(force: bool = True) -> Path:
    """Compile ref.c into a shared library with gcc (no fast-math, no FMA
    contraction, so every double operation is the one written)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fno-fast-math", "-fPIC", "-shared", str(_SRC), "-o", str(tmp),
                        "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path) -> C.CDLL:
    L = C.CDLL(str(path))
    P, I, I64 = C.c_void_p, C.c_int, C.c_int64
    L.ref_decode_fp8_e4m3fn.restype = C.c_double
    L.ref_decode_fp8_e4m3fn.argtypes = [C.c_uint8]
    L.ref_decode_e2m1.restype = C.c_double
    L.ref_decode_e2m1.argtypes = [C.c_uint8]
    L.ref_decode_ue8m0.restype = C.c_double
    L.ref_decode_ue8m0.argtypes = [C.c_uint8]
    L.ref_decode_bf16.restype = C.c_double
    L.ref_decode_bf16.argtypes = [C.c_uint16]
    L.ref_logits_dense.restype = None
    L.ref_logits_dense.argtypes = [P, I, P, P, P, I, P, P, I, I, I, P, I64]
    L.ref_logits_paged.restype = None
    L.ref_logits_paged.argtypes = [P, I, P, P, P, I, I, P, I64, P, P, I, I, I, P, I64]
    L.ref_logits_sparse.restype = None
    L.ref_logits_sparse.argtypes = [P, I, P, P, P, I, P, P, P, I64, P, I, I, I, I, P, I64]
    L.ref_logits_paged_sparse.restype = None
    L.ref_logits_paged_sparse.argtypes = [P, I, P, P, P, I, I, P, I64, P, P, P, I64, P, I, I, I, I, P, I64]
    L.ref_topk.restype = None
    L.ref_topk.argtypes = [P, I64, P, I64, I, I, P, P, I64]
    L.ref_encode_fp8_e4m3fn.argtypes = [C.c_float]
    L.ref_encode_fp8_e4m3fn.restype = C.c_uint8
    L.ref_encode_e2m1.argtypes = [C.c_double]
    L.ref_encode_e2m1.restype = C.c_uint8
    L.ref_kcache_write.argtypes = [P, I64, P, I, P, P, I64]
    L.ref_kcache_write.restype = I64
    L.ref_candidate_blocks.argtypes = [P, I64, P, I64, I, I, I, P, I64, P]
    L.ref_candidate_blocks.restype = None
    return L


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build(force=False)
        _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def variant(path):
    """Run the oracle functions against another build of ref.c (used by the tests that
    plant a mistake in a copy of the oracle and check that a pin catches it)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dt is None else a.astype(dt, copy=False))


def _shape_q(q):
    rows, heads, dim = q.shape
    return rows, heads, dim


# ------------------------------------------------------------------ decoding tables


def decode_fp8(codes) -> np.ndarray:
    L = lib()
    return np.array([L.ref_decode_fp8_e4m3fn(int(c)) for c in np.ravel(codes)]).reshape(np.shape(codes))


def decode_e2m1(nibbles) -> np.ndarray:
    L = lib()
    return np.array([L.ref_decode_e2m1(int(c)) for c in np.ravel(nibbles)]).reshape(np.shape(nibbles))


def decode_ue8m0(e) -> np.ndarray:
    L = lib()
    return np.array([L.ref_decode_ue8m0(int(c)) for c in np.ravel(e)]).reshape(np.shape(e))


def decode_bf16(bits) -> np.ndarray:
    L = lib()
    return np.array([L.ref_decode_bf16(int(c)) for c in np.ravel(bits)]).reshape(np.shape(bits))


# ------------------------------------------------------------------ Eq. (1) logits


def logits_dense(q, q_dtype, w, k, k_scale, k_dtype, row_ks, row_ke, ld=None) -> np.ndarray:
    """fp32 [rows, ld]: I(r, ks+c) for c < ke-ks, -inf beyond."""
    q, w, k = _c(q), _c(w, np.float32), _c(k)
    k_scale = _c(k_scale)
    row_ks, row_ke = _c(row_ks, np.int32), _c(row_ke, np.int32)
    rows, heads, dim = _shape_q(q)
    if ld is None:
        ld = int((row_ke - row_ks).max()) if rows else 0
    out = np.empty((rows, ld), np.float32)
    lib().ref_logits_dense(_p(q), DTYPES[q_dtype], _p(w), _p(k), _p(k_scale), DTYPES[k_dtype],
                           _p(row_ks), _p(row_ke), rows, heads, dim, _p(out), ld)
    return out


def logits_paged(q, q_dtype, w, k_pages, k_scale_pages, k_dtype, block_table, seq_lens,
                 row_req=None, ld=None) -> np.ndarray:
    """fp32 [rows, ld]: I(r, s) for logical positions s < seq_len, -inf beyond."""
    q, w, kp, sp = _c(q), _c(w, np.float32), _c(k_pages), _c(k_scale_pages)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    rr = _c(row_req, np.int32)
    rows, heads, dim = _shape_q(q)
    page = kp.shape[1]
    if ld is None:
        ld = bt.shape[1] * page
    out = np.empty((rows, ld), np.float32)
    lib().ref_logits_paged(_p(q), DTYPES[q_dtype], _p(w), _p(kp), _p(sp), DTYPES[k_dtype], page,
                           _p(bt), bt.shape[1], _p(sl), _p(rr), rows, heads, dim, _p(out), ld)
    return out


def logits_sparse(q, q_dtype, w, k, k_scale, k_dtype, row_ks, row_ke, cand, n_cols, block,
                  ld=None) -> np.ndarray:
    """fp32 [rows, ld] over sparse columns: column c is token cand[c//block]*block + c%block."""
    q, w, k, ks = _c(q), _c(w, np.float32), _c(k), _c(k_scale)
    row_ks, row_ke = _c(row_ks, np.int32), _c(row_ke, np.int32)
    cand, n_cols = _c(cand, np.int32), _c(n_cols, np.int32)
    rows, heads, dim = _shape_q(q)
    if ld is None:
        ld = cand.shape[1] * block
    out = np.empty((rows, ld), np.float32)
    lib().ref_logits_sparse(_p(q), DTYPES[q_dtype], _p(w), _p(k), _p(ks), DTYPES[k_dtype],
                            _p(row_ks), _p(row_ke), _p(cand), cand.shape[1], _p(n_cols), block,
                            rows, heads, dim, _p(out), ld)
    return out


def logits_paged_sparse(q, q_dtype, w, k_pages, k_scale_pages, k_dtype, block_table, seq_lens, cand, n_cols,
                        block, row_req=None, ld=None) -> np.ndarray:
    """fp32 [rows, ld] over candidate columns of paged rows: column c is the row's logical
    token cand[c//block]*block + c%block, read through the row's page table."""
    q, w, kp, sp = _c(q), _c(w, np.float32), _c(k_pages), _c(k_scale_pages)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    rr = _c(row_req, np.int32)
    cand, n_cols = _c(cand, np.int32), _c(n_cols, np.int32)
    rows, heads, dim = _shape_q(q)
    page = kp.shape[1]
    if ld is None:
        ld = cand.shape[1] * block
    out = np.empty((rows, ld), np.float32)
    lib().ref_logits_paged_sparse(_p(q), DTYPES[q_dtype], _p(w), _p(kp), _p(sp), DTYPES[k_dtype], page,
                                  _p(bt), bt.shape[1], _p(sl), _p(rr), _p(cand), cand.shape[1], _p(n_cols),
                                  block, rows, heads, dim, _p(out), ld)
    return out


# ------------------------------------------------------------------ selection


def topk(logits, k, lens=None):
    """Exact top-k per row: (idx int32 [rows, k], val fp32 [rows, k]), selection order,
    -1 / -inf padding. ``lens`` limits each row to its first lens[r] entries."""
    lg = _c(logits, np.float32)
    rows, ncols = lg.shape
    ln = _c(lens, np.int32)
    idx = np.empty((rows, k), np.int32)
    val = np.empty((rows, k), np.float32)
    lib().ref_topk(_p(lg), ncols, _p(ln), ncols, rows, k, _p(idx), _p(val), k)
    return idx, val


def candidate_blocks(logits, block, n_top, lens=None):
    """Candidate-source step of the two-level indexer: (cand int32 [rows, n_top], n_cand
    int32 [rows]). A block's score is the largest score of its tokens; the n_top best
    blocks (higher score first, equal scores by lower id) in ascending id, -1 padded.
    Row r covers its first lens[r] tokens (all columns when lens is None)."""
    lg = _c(logits, np.float32)
    rows, ncols = lg.shape
    ln = None if lens is None else _c(lens, np.int32)
    cand = np.empty((rows, n_top), np.int32)
    n_cand = np.empty(rows, np.int32)
    lib().ref_candidate_blocks(_p(lg), ncols, _p(ln), ncols, rows, block, n_top,
                               _p(cand), n_top, _p(n_cand))
    return cand, n_cand


def columns_to_tokens(col_idx, cand, block):
    """Map selected sparse columns to token positions (relative to the row start): column c
    of row r is token cand[r][c // block] * block + c % block (vLLM sparse_indexer page:
    sparse_indices hold block ids, col_indices the selected columns). -1 stays -1."""
    col_idx = np.asarray(col_idx)
    cand = np.asarray(cand)
    b = np.where(col_idx >= 0, col_idx // block, 0)
    tok = np.take_along_axis(cand, b, axis=1).astype(np.int64) * block + np.where(col_idx >= 0, col_idx % block, 0)
    return np.where(col_idx >= 0, tok, -1).astype(np.int32)


def select_case(case, k=None, with_logits=False):
    """Logits then top-k for a synth case (Dense / Paged / Sparse); the returned indices are
    key positions: relative to row_ks (dense), logical positions (paged) or token positions
    relative to row_ks (sparse)."""
    k = case.topk if k is None else k
    kind = type(case).__name__
    if kind == "Dense":
        lg = logits_dense(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                          case.row_ks, case.row_ke)
        idx, val = topk(lg, k)
    elif kind == "Paged":
        lg = logits_paged(case.q, case.q_dtype, case.w, case.k_pages, case.k_scale_pages,
                          case.k_dtype, case.block_table, case.seq_lens, case.row_req)
        idx, val = topk(lg, k)
    elif kind == "Sparse":
        lg = logits_sparse(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                           case.row_ks, case.row_ke, case.cand, case.n_cols, case.block)
        cidx, val = topk(lg, k)
        idx = columns_to_tokens(cidx, case.cand, case.block)
    elif kind == "PagedSparse":
        lg = logits_paged_sparse(case.q, case.q_dtype, case.w, case.k_pages, case.k_scale_pages, case.k_dtype,
                                 case.block_table, case.seq_lens, case.cand, case.n_cols, case.block,
                                 row_req=case.row_req)
        cidx, val = topk(lg, k)
        idx = columns_to_tokens(cidx, case.cand, case.block)
    else:
        raise TypeError(kind)
    return (idx, val, lg) if with_logits else (idx, val)


def subset_rows(case, rows):
    """The same case restricted to the given rows (for sampled checks at full size)."""
    import copy
    rows = np.asarray(rows)
    c = copy.copy(case)
    c.q = case.q[rows]
    c.w = case.w[rows]
    kind = type(case).__name__
    if kind in ("Dense", "Sparse"):
        c.row_ks = case.row_ks[rows]
        c.row_ke = case.row_ke[rows]
    if kind in ("Sparse", "PagedSparse"):
        c.cand = case.cand[rows]
        c.n_cols = case.n_cols[rows]
    if kind in ("Paged", "PagedSparse"):
        c.seq_lens = case.seq_lens[rows]
        if case.row_req is None:
            c.row_req = rows.astype(np.int32)
        else:
            c.row_req = case.row_req[rows]
    return c


def encode_fp8(y) -> np.ndarray:
    """e4m3fn codes of float32 values (nearest code, ties to even, saturating)."""
    y = np.asarray(y, np.float32)
    f = lib().ref_encode_fp8_e4m3fn
    return np.array([f(float(v)) for v in y.reshape(-1)], np.uint8).reshape(y.shape)


def encode_e2m1(v) -> np.ndarray:
    """e2m1 nibbles of values (nearest code, ties to even, saturating at 6)."""
    v = np.asarray(v, np.float64)
    f = lib().ref_encode_e2m1
    return np.array([f(float(x)) for x in v.reshape(-1)], np.uint8).reshape(v.shape)


def kcache_write(k_new_bf16, slot_mapping, k_dtype, cache, cache_scale):
    """Quantise new keys (bf16 bits [n, 128]) into ``cache`` / ``cache_scale`` (numpy
    arrays, updated in place) at their slots; returns the count of out-of-range slots.
    fp8: cache uint8 [n_slots, 128], cache_scale float32 [n_slots]; MXFP4: cache uint8
    [n_slots, 64], cache_scale uint8 [n_slots, 4]."""
    kd = DTYPES[k_dtype]
    k_new = _c(k_new_bf16, np.uint16)
    slots = _c(slot_mapping, np.int64)
    assert cache.flags.c_contiguous and cache_scale.flags.c_contiguous
    return int(lib().ref_kcache_write(_p(k_new), k_new.shape[0], _p(slots), kd, _p(cache), _p(cache_scale),
                                      cache.shape[0]))


# ------------------------------------------------------------------ sparse attention

_BF16_TABLE = None


def _bf16_table() -> np.ndarray:
    """float64 value of every bf16 bit pattern, from the decoder above."""
    global _BF16_TABLE
    if _BF16_TABLE is None:
        _BF16_TABLE = decode_bf16(np.arange(65536, dtype=np.uint32)).astype(np.float64)
    return _BF16_TABLE


def sparse_attn_paged(q_bits, kv_bits, block_table, seq_lens, indices, scale, row_req=None, page_size=64):
    """The attention of Eq. (2) over the selected entries (DeepSeek-V3.2 architecture
    section: the output attends only the key-value entries whose index scores are in the
    row's top-k), in MLA's single-shared-entry form: every token keeps one 576-element
    entry c_s, shared by all heads; head h scores it as scale * (q_h . c_s) and reads its
    first 512 elements as the value (the 512- and 576-element vectors of the llama.cpp
    thread). Plain numpy in float64.

    q_bits [rows, H, 576] and kv_bits [n_pages, page_size, 576] are bf16 bit patterns
    (uint16); row r's logical position s lives in page block_table[req(r)][s // page_size],
    slot s % page_size. indices [rows, k]: logical positions, -1 (or any position outside
    [0, seq_lens[r])) is skipped. Returns (out float32 [rows, H, 512], lse float32
    [rows, H]): out = sum_i p_i c_{s_i}[:512] with p the softmax of the scores over the
    valid selected entries; lse = log sum_i exp(score_i); a row with no valid entry gets
    out = 0 and lse = -inf."""
    tab = _bf16_table()
    q = tab[np.asarray(q_bits, np.uint16)]
    kv = np.asarray(kv_bits, np.uint16)
    bt = np.asarray(block_table)
    idx = np.asarray(indices)
    rows, H, D = q.shape
    out = np.zeros((rows, H, 512), np.float64)
    lse = np.full((rows, H), -np.inf, np.float64)
    for r in range(rows):
        req = r if row_req is None else int(row_req[r])
        pos = [int(s) for s in idx[r] if 0 <= s < seq_lens[r]]
        if not pos:
            continue
        c = np.stack([tab[kv[bt[req][s // page_size], s % page_size]] for s in pos])
        z = scale * (q[r] @ c.T)                   # [H, n]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        den = e.sum(axis=1, keepdims=True)
        out[r] = (e / den) @ c[:, :512]
        lse[r] = (m + np.log(den))[:, 0]
    return out.astype(np.float32), lse.astype(np.float32)
