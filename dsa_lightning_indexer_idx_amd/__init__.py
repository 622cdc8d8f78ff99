"""dsaidx: the DeepSeek Sparse Attention lightning indexer (scores + exact top-k) on
AMD Instinct MI355X (gfx950).

This module is a thin ctypes binding over the C ABI declared in ``include/dsaidx.h``
and implemented by ``libdsaidx.so`` (hand-written HIP kernels). It only marshals
arguments: torch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels. The functions carry the C names.

The library is loaded on first use; if it has not been built, the call raises
``RuntimeError`` (there is no fallback path).
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

_LIB_PATH = Path(__file__).resolve().parent / "libdsaidx.so"

IDX_OK, IDX_ERR_ARG, IDX_ERR_UNSUPPORTED, IDX_ERR_WORKSPACE, IDX_ERR_HIP = 0, 1, 2, 3, 4
IDX_BF16, IDX_FP8_E4M3, IDX_MXFP4 = 1, 2, 3
IDX_MODE_DENSE, IDX_MODE_PAGED, IDX_MODE_SPARSE_BLOCKS, IDX_MODE_PREFILL, IDX_MODE_PAGED_SPARSE_BLOCKS = 1, 2, 3, 4, 5
IDX_TOPK_UNSORTED = 1
IDX_SELECT_NO_CUTOFF = 2
IDX_SELECT_ONE_PASS = 4
IDX_DEVERR_RANGE, IDX_DEVERR_PAGE, IDX_DEVERR_BLOCK, IDX_DEVERR_SLOT, IDX_DEVERR_ORDER = 1, 2, 4, 8, 16
IDX_HEADS, IDX_DIM, IDX_MAX_K = 64, 128, 2048
IDX_NOALLOC_SCRATCH_BYTES = 128 << 20

KDTYPES = {"bf16": IDX_BF16, "fp8": IDX_FP8_E4M3, "mxfp4": IDX_MXFP4}

# Every symbol include/dsaidx.h declares.
EXPORTS = ("idx_logits", "idx_logits_prefill", "idx_logits_paged", "idx_logits_paged_sparse_blocks", "idx_logits_sparse_blocks", "idx_topk",
           "idx_topk_workspace", "idx_select", "idx_select_workspace", "idx_status_string",
           "idx_last_error", "idx_version", "idx_device_errors", "idx_kcache_write", "idx_read_probe",
           "idx_candidate_blocks", "idx_candidate_blocks_workspace", "idx_sparse_attn_paged",
           "idx_sparse_attn_workspace", "idx_select_noalloc")


class IdxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_STATUS_NAMES = {0: "IDX_OK", 1: "IDX_ERR_ARG", 2: "IDX_ERR_UNSUPPORTED",
                 3: "IDX_ERR_WORKSPACE", 4: "IDX_ERR_HIP"}


class idx_problem(C.Structure):
    """Mirror of ``struct idx_problem`` (include/dsaidx.h)."""
    _fields_ = [
        ("mode", C.c_int32), ("rows", C.c_int32),
        ("q", C.c_void_p), ("q_dtype", C.c_int32), ("k_dtype", C.c_int32),
        ("w", C.c_void_p), ("k", C.c_void_p), ("k_scale", C.c_void_p),
        ("n_keys", C.c_int64),
        ("row_ks", C.c_void_p), ("row_ke", C.c_void_p),
        ("max_cols", C.c_int64),
        ("page_size", C.c_int32), ("block_size", C.c_int32),
        ("block_table", C.c_void_p), ("bt_rows", C.c_int64), ("bt_ld", C.c_int64),
        ("seq_lens", C.c_void_p), ("row_req", C.c_void_p),
        ("cand_blocks", C.c_void_p), ("cand_ld", C.c_int64), ("n_cols", C.c_void_p),
    ]


_lib = None


def library_path() -> Path:
    return _LIB_PATH


def lib() -> C.CDLL:
    """The loaded libdsaidx.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m dsa_lightning_indexer_idx_amd.build")
        L = C.CDLL(str(_LIB_PATH))
        P, I, I64, U32, SZ = C.c_void_p, C.c_int, C.c_int64, C.c_uint32, C.c_size_t
        L.idx_logits.argtypes = [P, I, P, P, P, I, I64, P, P, I, P, I64, P]
        L.idx_logits_prefill.argtypes = [P, I, P, P, P, I, I64, P, P, I, P, I64, P]
        L.idx_logits_paged.argtypes = [P, I, P, P, P, I, I64, I, P, I64, I64, P, P, I, P, I64, P]
        L.idx_logits_sparse_blocks.argtypes = [P, I, P, P, P, I, I64, P, P, P, I64, P, I, I, P, I64, P]
        L.idx_logits_paged_sparse_blocks.argtypes = [P, I, P, P, P, I, I64, I, P, I64, I64, P, P, P, I64, P, I,
                                                     I, P, I64, P]
        L.idx_topk.argtypes = [P, I64, P, I64, I, I, P, P, I64, U32, P, SZ, P]
        L.idx_topk_workspace.argtypes = [I, I64, I]
        L.idx_topk_workspace.restype = SZ
        L.idx_select.argtypes = [C.POINTER(idx_problem), I, P, P, I64, U32, P, SZ, P]
        L.idx_select_noalloc.argtypes = [C.POINTER(idx_problem), I, P, P, I64, U32, P]
        L.idx_select_workspace.argtypes = [C.POINTER(idx_problem), I]
        L.idx_select_workspace.restype = SZ
        L.idx_status_string.argtypes = [I]
        L.idx_status_string.restype = C.c_char_p
        L.idx_last_error.argtypes = []
        L.idx_last_error.restype = C.c_char_p
        L.idx_version.restype = I
        L.idx_device_errors.argtypes = [P]
        L.idx_device_errors.restype = I
        L.idx_read_probe.argtypes = [P, SZ, P, P]
        L.idx_kcache_write.argtypes = [P, I, I64, P, P, P, I, I64, P]
        L.idx_candidate_blocks.argtypes = [P, I64, P, I64, I, I, I, P, I64, P, P, SZ, P]
        L.idx_candidate_blocks_workspace.argtypes = [I, I64]
        L.idx_candidate_blocks_workspace.restype = SZ
        L.idx_sparse_attn_paged.argtypes = [P, I, P, I64, I, P, I64, I64, P, P, P, I64, I, I, C.c_float, P, P,
                                            P, SZ, P]
        L.idx_sparse_attn_workspace.argtypes = [I, I, I]
        L.idx_sparse_attn_workspace.restype = SZ
        for name in ("idx_logits", "idx_logits_paged", "idx_logits_sparse_blocks", "idx_topk",
                     "idx_select", "idx_read_probe", "idx_kcache_write", "idx_candidate_blocks",
                     "idx_sparse_attn_paged"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != IDX_OK:
        raise IdxError(status, lib().idx_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


# Shape checks of the binding: the kernels take plain pointers and trust the sizes they
# are given, so a tensor that is on the host, strided or smaller than its role needs is
# rejected here rather than read or written out of bounds on the device.
_HEADS, _DIM = 64, 128
_KEY_BYTES = {"fp8": 128, "bf16": 256, "mxfp4": 64}  # one key row
_SCALE_BYTES = {"fp8": 4, "mxfp4": 4}                 # one key's scale(s)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need(t, name, dtype=None, numel=None, min_numel=None, nbytes=None):
    """``t`` (or None) as a contiguous device tensor of the given dtype and size."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")
    if nbytes is not None and _nbytes(t) != nbytes:
        raise ValueError(f"{name} has {_nbytes(t)} bytes, expected {nbytes}")
    return t


def _rows_out(t, name, rows, dtype, min_cols):
    """A [rows, >= min_cols] output matrix; returns its column count."""
    _need(t, name, dtype)
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < min_cols:
        raise ValueError(f"{name} must be [{rows}, >= {min_cols}], got {list(t.shape)}")
    return t.shape[1]


def _check_score_inputs(q, w, k, k_scale, k_dtype, n_tokens):
    """q [rows, 64, 128] (fp8 bytes or bf16), w fp32 [rows, 64], key rows and scales of
    n_tokens tokens in the layout of k_dtype; returns rows."""
    import torch
    if k_dtype not in _KEY_BYTES:
        raise ValueError(f"k_dtype must be one of {sorted(_KEY_BYTES)}, got {k_dtype!r}")
    rows = q.shape[0]
    _need(q, "q", nbytes=rows * _HEADS * _DIM * (2 if k_dtype == "bf16" else 1))
    _need(w, "w", torch.float32, numel=rows * _HEADS)
    _need(k, "k", nbytes=n_tokens * _KEY_BYTES[k_dtype])
    if k_dtype == "bf16":
        _need(k_scale, "k_scale")
    else:
        if k_scale is None:
            raise ValueError(f"k_scale is required for {k_dtype} keys")
        _need(k_scale, "k_scale", nbytes=n_tokens * _SCALE_BYTES[k_dtype])
    return rows


def _workspace_bytes(workspace) -> int:
    if workspace is None:
        return 0
    _need(workspace, "workspace")
    return _nbytes(workspace)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _q_dtype(k_dtype: str) -> int:
    return IDX_BF16 if k_dtype == "bf16" else IDX_FP8_E4M3


# ----------------------------------------------------------------------------- scores


def idx_logits(q, w, k, k_scale, row_ks, row_ke, *, k_dtype: str, ld: int | None = None,
               out=None, stream=None, prefill: bool = False):
    """Scores of rows over contiguous key ranges (C: idx_logits, or idx_logits_prefill when
    ``prefill``: the rows are one prefill chunk's queries sharing the key array). Returns
    fp32 [rows, ld]."""
    import torch
    rows = _check_score_inputs(q, w, k, k_scale, k_dtype, k.shape[0])
    _need(row_ks, "row_ks", torch.int32, numel=rows)
    _need(row_ke, "row_ke", torch.int32, numel=rows)
    if out is None:
        if ld is None:
            raise ValueError("give ld or out")
        out = torch.empty((rows, ld), dtype=torch.float32, device=q.device)
    ld = _rows_out(out, "out", rows, torch.float32, 1)
    fn = lib().idx_logits_prefill if prefill else lib().idx_logits
    _check(fn(_ptr(q), _q_dtype(k_dtype), _ptr(w), _ptr(k), _ptr(k_scale), KDTYPES[k_dtype], k.shape[0],
              _ptr(row_ks), _ptr(row_ke), rows, _ptr(out), ld, _stream(stream)))
    return out


def _check_paged_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req, k_dtype):
    """Paged score inputs: k_pages [n_pages, page_size, key bytes]; returns (rows,
    page_size, bt_rows, bt_ld)."""
    import torch
    if k_pages.dim() < 2:
        raise ValueError("k_pages must be [n_pages, page_size, ...]")
    page = k_pages.shape[1]
    rows = _check_score_inputs(q, w, k_pages, k_scale_pages, k_dtype, k_pages.shape[0] * page)
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [bt_rows, bt_ld]")
    _need(seq_lens, "seq_lens", torch.int32, min_numel=rows)
    _need(row_req, "row_req", torch.int32, numel=rows)
    return rows, page, block_table.shape[0], block_table.shape[1]


def idx_logits_paged(q, w, k_pages, k_scale_pages, block_table, seq_lens, *, k_dtype: str,
                     row_req=None, ld: int | None = None, out=None, stream=None):
    """Scores of rows over a paged key cache (C: idx_logits_paged)."""
    import torch
    rows, page, bt_rows, bt_ld = _check_paged_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens,
                                                     row_req, k_dtype)
    if out is None:
        ld = bt_ld * page if ld is None else ld
        out = torch.empty((rows, ld), dtype=torch.float32, device=q.device)
    _rows_out(out, "out", rows, torch.float32, 1)
    _check(lib().idx_logits_paged(_ptr(q), _q_dtype(k_dtype), _ptr(w), _ptr(k_pages),
                                  _ptr(k_scale_pages), KDTYPES[k_dtype], k_pages.shape[0], page,
                                  _ptr(block_table), bt_rows, bt_ld, _ptr(seq_lens),
                                  _ptr(row_req), rows, _ptr(out), out.shape[1],
                                  _stream(stream)))
    return out


def _check_sparse_inputs(q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols, k_dtype):
    """Candidate-block score inputs; returns (rows, cand_ld)."""
    import torch
    rows = _check_score_inputs(q, w, k, k_scale, k_dtype, k.shape[0])
    _need(row_ks, "row_ks", torch.int32, numel=rows)
    _need(row_ke, "row_ke", torch.int32, numel=rows)
    _need(cand_blocks, "cand_blocks", torch.int32)
    if cand_blocks.dim() != 2 or cand_blocks.shape[0] != rows:
        raise ValueError(f"cand_blocks must be [{rows}, cand_ld]")
    _need(n_cols, "n_cols", torch.int32, numel=rows)
    return rows, cand_blocks.shape[1]


def idx_logits_sparse_blocks(q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols, *,
                             k_dtype: str, block_size: int = 128, ld: int | None = None,
                             out=None, stream=None):
    """Scores of two-level rows over their candidate blocks (C: idx_logits_sparse_blocks)."""
    import torch
    rows, cand_ld = _check_sparse_inputs(q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols, k_dtype)
    if out is None:
        ld = cand_ld * block_size if ld is None else ld
        out = torch.empty((rows, ld), dtype=torch.float32, device=q.device)
    _rows_out(out, "out", rows, torch.float32, 1)
    _check(lib().idx_logits_sparse_blocks(_ptr(q), _q_dtype(k_dtype), _ptr(w), _ptr(k),
                                          _ptr(k_scale), KDTYPES[k_dtype], k.shape[0],
                                          _ptr(row_ks), _ptr(row_ke), _ptr(cand_blocks), cand_ld,
                                          _ptr(n_cols), block_size, rows, _ptr(out),
                                          out.shape[1], _stream(stream)))
    return out


def _check_paged_sparse_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req, cand_blocks, n_cols,
                               k_dtype):
    """Paged candidate-block score inputs; returns (rows, page_size, bt_rows, bt_ld, cand_ld)."""
    import torch
    rows, page, bt_rows, bt_ld = _check_paged_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens,
                                                     row_req, k_dtype)
    _need(cand_blocks, "cand_blocks", torch.int32)
    if cand_blocks.dim() != 2 or cand_blocks.shape[0] != rows:
        raise ValueError(f"cand_blocks must be [{rows}, cand_ld]")
    _need(n_cols, "n_cols", torch.int32, numel=rows)
    return rows, page, bt_rows, bt_ld, cand_blocks.shape[1]


def idx_logits_paged_sparse_blocks(q, w, k_pages, k_scale_pages, block_table, seq_lens, cand_blocks, n_cols, *,
                                   k_dtype: str, block_size: int = 128, row_req=None, ld: int | None = None,
                                   out=None, stream=None):
    """Scores of two-level decode rows over their candidate blocks in a paged cache
    (C: idx_logits_paged_sparse_blocks)."""
    import torch
    rows, page, bt_rows, bt_ld, cand_ld = _check_paged_sparse_inputs(q, w, k_pages, k_scale_pages, block_table,
                                                                     seq_lens, row_req, cand_blocks, n_cols, k_dtype)
    if out is None:
        ld = cand_ld * block_size if ld is None else ld
        out = torch.empty((rows, ld), dtype=torch.float32, device=q.device)
    _rows_out(out, "out", rows, torch.float32, 1)
    _check(lib().idx_logits_paged_sparse_blocks(_ptr(q), _q_dtype(k_dtype), _ptr(w), _ptr(k_pages),
                                                _ptr(k_scale_pages), KDTYPES[k_dtype], k_pages.shape[0], page,
                                                _ptr(block_table), bt_rows, bt_ld, _ptr(seq_lens), _ptr(row_req),
                                                _ptr(cand_blocks), cand_ld, _ptr(n_cols), block_size, rows,
                                                _ptr(out), out.shape[1], _stream(stream)))
    return out


# ----------------------------------------------------------------------------- selection


def idx_topk_workspace(rows: int, n_cols: int, k: int) -> int:
    return int(lib().idx_topk_workspace(rows, n_cols, k))


def idx_topk(logits, k: int, *, lens=None, n_cols: int | None = None, sorted: bool = True,
             values: bool = True, out_idx=None, out_val=None, workspace=None, stream=None):
    """Exact top-k per row (C: idx_topk). Returns (idx int32 [rows, k], val fp32 or None)."""
    import torch
    _need(logits, "logits", torch.float32)
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, ld]")
    rows, ld = logits.shape
    _need(lens, "lens", torch.int32, min_numel=rows)
    n_cols = ld if n_cols is None else n_cols
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=logits.device)
    if values and out_val is None:
        out_val = torch.empty((rows, k), dtype=torch.float32, device=logits.device)
    _rows_out(out_idx, "out_idx", rows, torch.int32, k)
    if out_val is not None and (_rows_out(out_val, "out_val", rows, torch.float32, k) != out_idx.shape[1]):
        raise ValueError("out_val must have the shape of out_idx")
    need = idx_topk_workspace(rows, n_cols, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    wsb = _workspace_bytes(workspace)
    _check(lib().idx_topk(_ptr(logits), ld, _ptr(lens), n_cols, rows, k, _ptr(out_idx),
                          _ptr(out_val), out_idx.shape[1], 0 if sorted else IDX_TOPK_UNSORTED,
                          _ptr(workspace), wsb, _stream(stream)))
    return out_idx, out_val


def idx_candidate_blocks_workspace(rows: int, n_cols: int) -> int:
    return int(lib().idx_candidate_blocks_workspace(rows, n_cols))


def idx_candidate_blocks(logits, block_size: int, n_top: int, *, lens=None, n_cols: int | None = None,
                         cand=None, n_cand=None, workspace=None, stream=None):
    """Candidate blocks of each row (C: idx_candidate_blocks). Returns (cand int32
    [rows, n_top] ascending block ids, -1 padded; n_cand int32 [rows]). ``logits`` may be
    a view of whole rows of a wider matrix (unit column stride; ld = its row stride)."""
    import torch
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be 2-D with unit column stride")
    if not logits.is_cuda or logits.dtype != torch.float32:
        raise ValueError("logits must be a float32 device tensor")
    rows = logits.shape[0]
    _need(lens, "lens", torch.int32, min_numel=rows)
    ld = max(logits.stride(0), logits.shape[1], 1)
    n_cols = logits.shape[1] if n_cols is None else n_cols
    if n_cols > logits.shape[1]:
        raise ValueError(f"n_cols = {n_cols} exceeds the {logits.shape[1]} columns of logits")
    if cand is None:
        cand = torch.empty((rows, n_top), dtype=torch.int32, device=logits.device)
    if n_cand is None:
        n_cand = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _rows_out(cand, "cand", rows, torch.int32, n_top)
    _need(n_cand, "n_cand", torch.int32, min_numel=rows)
    need = idx_candidate_blocks_workspace(rows, n_cols)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    wsb = _workspace_bytes(workspace)
    _check(lib().idx_candidate_blocks(_ptr(logits), ld, _ptr(lens), n_cols, rows, block_size, n_top,
                                      _ptr(cand), cand.shape[1], _ptr(n_cand), _ptr(workspace), wsb,
                                      _stream(stream)))
    return cand, n_cand


def idx_sparse_attn_workspace(rows: int, heads: int, k: int) -> int:
    return int(lib().idx_sparse_attn_workspace(rows, heads, k))


def idx_sparse_attn_paged(q, kv_pages, block_table, seq_lens, indices, scale: float, *, k: int | None = None,
                          row_req=None, out=None, lse=None, with_lse: bool = True, workspace=None, stream=None):
    """Attention over each row's selected entries (C: idx_sparse_attn_paged). q bf16
    [rows, heads, 576]; kv_pages bf16 [n_pages, 64, 576]; indices int32 [rows, >= k].
    Returns (out fp32 [rows, heads, 512], lse fp32 [rows, heads] or None)."""
    import torch
    if q.dim() != 3 or kv_pages.dim() < 2 or block_table.dim() != 2 or indices.dim() != 2:
        raise ValueError("q must be [rows, heads, 576], kv_pages [n_pages, 64, 576], block_table and "
                         "indices 2-D")
    rows, heads, _ = q.shape
    _need(q, "q", nbytes=rows * heads * 576 * 2)
    _need(kv_pages, "kv_pages", nbytes=kv_pages.shape[0] * kv_pages.shape[1] * 576 * 2)
    _need(block_table, "block_table", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32, min_numel=rows)
    _need(indices, "indices", torch.int32)
    if indices.shape[0] != rows:
        raise ValueError(f"indices must have {rows} rows")
    _need(row_req, "row_req", torch.int32, numel=rows)
    k = indices.shape[1] if k is None else k
    if out is None:
        out = torch.empty((rows, heads, 512), dtype=torch.float32, device=q.device)
    if with_lse and lse is None:
        lse = torch.empty((rows, heads), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, numel=rows * heads * 512)
    _need(lse, "lse", torch.float32, numel=rows * heads)
    need = idx_sparse_attn_workspace(rows, heads, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = _workspace_bytes(workspace)
    _check(lib().idx_sparse_attn_paged(_ptr(q), heads, _ptr(kv_pages), kv_pages.shape[0], kv_pages.shape[1],
                                       _ptr(block_table), block_table.shape[0], block_table.shape[1],
                                       _ptr(seq_lens), _ptr(row_req), _ptr(indices), indices.shape[1], k, rows,
                                       float(scale), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                                       _stream(stream)))
    return out, lse


class Problem:
    """An ``idx_problem`` plus references that keep its tensors alive."""

    def __init__(self, st: idx_problem, tensors):
        self.st = st
        self._keep = tensors

    @property
    def rows(self) -> int:
        return self.st.rows


def dense_problem(q, w, k, k_scale, row_ks, row_ke, *, k_dtype: str, max_cols: int,
                  prefill: bool = False) -> Problem:
    """idx_logits arguments (IDX_MODE_DENSE), or with ``prefill`` idx_logits_prefill's
    (IDX_MODE_PREFILL: one prefill chunk's queries sharing the key array)."""
    import torch
    rows = _check_score_inputs(q, w, k, k_scale, k_dtype, k.shape[0])
    _need(row_ks, "row_ks", torch.int32, numel=rows)
    _need(row_ke, "row_ke", torch.int32, numel=rows)
    st = idx_problem(mode=IDX_MODE_PREFILL if prefill else IDX_MODE_DENSE, rows=q.shape[0], q=q.data_ptr(),
                     q_dtype=_q_dtype(k_dtype), k_dtype=KDTYPES[k_dtype], w=w.data_ptr(),
                     k=k.data_ptr(), k_scale=None if k_scale is None else k_scale.data_ptr(),
                     n_keys=k.shape[0], row_ks=row_ks.data_ptr(), row_ke=row_ke.data_ptr(),
                     max_cols=max_cols)
    return Problem(st, (q, w, k, k_scale, row_ks, row_ke))


def paged_problem(q, w, k_pages, k_scale_pages, block_table, seq_lens, *, k_dtype: str,
                  row_req=None) -> Problem:
    _check_paged_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req, k_dtype)
    st = idx_problem(mode=IDX_MODE_PAGED, rows=q.shape[0], q=q.data_ptr(),
                     q_dtype=_q_dtype(k_dtype), k_dtype=KDTYPES[k_dtype], w=w.data_ptr(),
                     k=k_pages.data_ptr(), k_scale=k_scale_pages.data_ptr(),
                     n_keys=k_pages.shape[0], page_size=k_pages.shape[1],
                     block_table=block_table.data_ptr(), bt_rows=block_table.shape[0],
                     bt_ld=block_table.shape[1], seq_lens=seq_lens.data_ptr(),
                     row_req=None if row_req is None else row_req.data_ptr())
    return Problem(st, (q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req))


def sparse_problem(q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols, *, k_dtype: str,
                   block_size: int = 128) -> Problem:
    _check_sparse_inputs(q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols, k_dtype)
    st = idx_problem(mode=IDX_MODE_SPARSE_BLOCKS, rows=q.shape[0], q=q.data_ptr(),
                     q_dtype=_q_dtype(k_dtype), k_dtype=KDTYPES[k_dtype], w=w.data_ptr(),
                     k=k.data_ptr(), k_scale=k_scale.data_ptr(), n_keys=k.shape[0],
                     row_ks=row_ks.data_ptr(), row_ke=row_ke.data_ptr(),
                     cand_blocks=cand_blocks.data_ptr(), cand_ld=cand_blocks.shape[1],
                     n_cols=n_cols.data_ptr(), block_size=block_size)
    return Problem(st, (q, w, k, k_scale, row_ks, row_ke, cand_blocks, n_cols))


def paged_sparse_problem(q, w, k_pages, k_scale_pages, block_table, seq_lens, cand_blocks, n_cols, *,
                         k_dtype: str, block_size: int = 128, row_req=None) -> Problem:
    _check_paged_sparse_inputs(q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req, cand_blocks, n_cols,
                               k_dtype)
    st = idx_problem(mode=IDX_MODE_PAGED_SPARSE_BLOCKS, rows=q.shape[0], q=q.data_ptr(),
                     q_dtype=_q_dtype(k_dtype), k_dtype=KDTYPES[k_dtype], w=w.data_ptr(),
                     k=k_pages.data_ptr(), k_scale=k_scale_pages.data_ptr(),
                     n_keys=k_pages.shape[0], page_size=k_pages.shape[1],
                     block_table=block_table.data_ptr(), bt_rows=block_table.shape[0],
                     bt_ld=block_table.shape[1], seq_lens=seq_lens.data_ptr(),
                     row_req=None if row_req is None else row_req.data_ptr(),
                     cand_blocks=cand_blocks.data_ptr(), cand_ld=cand_blocks.shape[1],
                     n_cols=n_cols.data_ptr(), block_size=block_size)
    return Problem(st, (q, w, k_pages, k_scale_pages, block_table, seq_lens, row_req, cand_blocks, n_cols))


def idx_select_workspace(problem: Problem, k: int) -> int:
    return int(lib().idx_select_workspace(C.byref(problem.st), k))


def idx_select(problem: Problem, k: int, *, sorted: bool = True, values: bool = True,
               out_idx=None, out_val=None, workspace=None, cutoff: bool = True, one_pass: bool = False,
               stream=None):
    """Scores + exact top-k in one call (C: idx_select). Returns (idx, val or None).
    cutoff=False sets IDX_SELECT_NO_CUTOFF (every scored entry goes to the exact finish);
    one_pass=True sets IDX_SELECT_ONE_PASS (the one-pass selection wherever it can run)."""
    import torch
    dev = problem._keep[0].device
    rows = problem.rows
    if out_idx is None:
        out_idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    if values and out_val is None:
        out_val = torch.empty((rows, k), dtype=torch.float32, device=dev)
    _rows_out(out_idx, "out_idx", rows, torch.int32, k)
    if out_val is not None and (_rows_out(out_val, "out_val", rows, torch.float32, k) != out_idx.shape[1]):
        raise ValueError("out_val must have the shape of out_idx")
    if workspace is None:
        workspace = torch.empty(max(idx_select_workspace(problem, k), 1), dtype=torch.uint8,
                                device=dev)
    wsb = _workspace_bytes(workspace)
    _check(lib().idx_select(C.byref(problem.st), k, _ptr(out_idx), _ptr(out_val),
                            out_idx.shape[1],
                            (0 if sorted else IDX_TOPK_UNSORTED) | (0 if cutoff else IDX_SELECT_NO_CUTOFF)
                            | (IDX_SELECT_ONE_PASS if one_pass else 0),
                            _ptr(workspace), wsb, _stream(stream)))
    return out_idx, out_val


def idx_select_noalloc(problem: Problem, k: int, *, sorted: bool = True, out_idx, out_val=None,
                       cutoff: bool = True, stream=None):
    """idx_select on the library's static device scratch (C: idx_select_noalloc): the C call
    allocates nothing; the caller passes the outputs. Returns (out_idx, out_val)."""
    import torch
    rows = problem.rows
    _rows_out(out_idx, "out_idx", rows, torch.int32, k)
    if out_val is not None and (_rows_out(out_val, "out_val", rows, torch.float32, k) != out_idx.shape[1]):
        raise ValueError("out_val must have the shape of out_idx")
    _check(lib().idx_select_noalloc(C.byref(problem.st), k, _ptr(out_idx), _ptr(out_val), out_idx.shape[1],
                                    (0 if sorted else IDX_TOPK_UNSORTED) | (0 if cutoff else IDX_SELECT_NO_CUTOFF),
                                    _stream(stream)))
    return out_idx, out_val


# ----------------------------------------------------------------------------- misc


def idx_version() -> int:
    return int(lib().idx_version())


def idx_kcache_write(k_new, slot_mapping, k_cache, k_scale, k_dtype="fp8", stream=None) -> None:
    """Quantise new keys (bf16 [n, 128]) into the key cache at their slots (int64 [n];
    negative = skip). fp8: k_cache uint8 with 128 bytes per slot (e.g. [pages, page, 128])
    and k_scale float32 with one per slot; MXFP4: 64 bytes and 4 UE8M0 bytes per slot."""
    import torch
    if k_dtype not in ("fp8", "mxfp4"):
        raise ValueError(f"k_dtype must be 'fp8' or 'mxfp4', got {k_dtype!r}")
    _need(k_new, "k_new", torch.bfloat16)
    if k_new.shape[-1] != 128:
        raise ValueError("k_new must be [n, 128]")
    n_new = k_new.numel() // 128
    _need(slot_mapping, "slot_mapping", torch.int64, numel=n_new)
    kd = {"fp8": IDX_FP8_E4M3, "mxfp4": IDX_MXFP4}[k_dtype]
    row = 128 if kd == IDX_FP8_E4M3 else 64
    _need(k_cache, "k_cache")
    n_slots = _nbytes(k_cache) // row
    _need(k_scale, "k_scale", min_numel=0)
    if _nbytes(k_scale) < n_slots * 4:
        raise ValueError(f"k_scale holds {_nbytes(k_scale)} bytes, {n_slots * 4} needed for {n_slots} slots")
    _check(lib().idx_kcache_write(_ptr(k_new), IDX_BF16, n_new, _ptr(slot_mapping), _ptr(k_cache),
                                  _ptr(k_scale), kd, n_slots, _stream(stream)))


def idx_read_probe(buf, sink, stream=None) -> None:
    """Read the whole device tensor ``buf`` once and discard it (a bandwidth probe);
    ``sink`` is a one-element int32 device tensor the probe may write."""
    import torch
    _need(buf, "buf")
    _need(sink, "sink", torch.int32, min_numel=1)
    _check(lib().idx_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def idx_device_errors(stream=None) -> int:
    v = int(lib().idx_device_errors(_stream(stream)))
    if v < 0:
        raise IdxError(IDX_ERR_HIP, lib().idx_last_error().decode())
    return v
