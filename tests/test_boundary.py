"""The C-ABI boundary on the CPU: the library loads, exports every symbol the header
declares, lays out idx_problem as the C compiler does, and rejects every argument the
host can check before anything touches a device (no GPU needed: these calls return
before the first HIP call)."""
import ctypes as C
import re
import subprocess
from pathlib import Path

import pytest

import dsa_lightning_indexer_idx_amd as D

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "dsaidx.h"

# Fake, aligned, never-dereferenced device addresses.
P = 0x10000
Q, W, K, S, KS, KE, OUT, BT, SL, CAND, NC, WS = (P * (i + 1) for i in range(12))


@pytest.fixture(scope="module")
def L():
    if not D.library_path().exists():
        from dsa_lightning_indexer_idx_amd import build
        build.build()
    return D.lib()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(idx_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(D.EXPORTS)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
    nm = subprocess.run(["nm", "-D", "--defined-only", str(D.library_path())], capture_output=True,
                        text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, re.M), f"{n} is not a defined text symbol"


def test_problem_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in D.idx_problem._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "dsaidx.h"\nint main(void){\n'
                   + "".join(f'printf("%zu\\n", offsetof(idx_problem, {f}));\n' for f in fields)
                   + 'printf("%zu\\n", sizeof(idx_problem));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [getattr(D.idx_problem, f).offset for f in fields] + [C.sizeof(D.idx_problem)]
    assert got == want


def test_misc_entry_points(L):
    assert L.idx_version() == 100
    assert L.idx_status_string(0) == b"IDX_OK"
    assert L.idx_status_string(3) == b"IDX_ERR_WORKSPACE"
    assert L.idx_topk_workspace(4096, 8192, 2048) == 0       # short rows: no workspace
    assert L.idx_topk_workspace(64, 131072, 2048) > 0        # long rows: histogram + lists


def _dense(L, **kw):
    a = dict(q=Q, qd=D.IDX_FP8_E4M3, w=W, k=K, sc=S, kd=D.IDX_FP8_E4M3, n=4096, ks=KS, ke=KE,
             rows=4, out=OUT, ld=4096)
    a.update(kw)
    return L.idx_logits(a["q"], a["qd"], a["w"], a["k"], a["sc"], a["kd"], a["n"], a["ks"], a["ke"],
                        a["rows"], a["out"], a["ld"], None)


def _paged(L, **kw):
    a = dict(q=Q, qd=D.IDX_FP8_E4M3, w=W, k=K, sc=S, kd=D.IDX_FP8_E4M3, npages=100, page=64, bt=BT,
             bt_rows=4, bt_ld=16, sl=SL, rr=None, rows=4, out=OUT, ld=1024)
    a.update(kw)
    return L.idx_logits_paged(a["q"], a["qd"], a["w"], a["k"], a["sc"], a["kd"], a["npages"],
                              a["page"], a["bt"], a["bt_rows"], a["bt_ld"], a["sl"], a["rr"],
                              a["rows"], a["out"], a["ld"], None)


def _sparse(L, **kw):
    a = dict(q=Q, qd=D.IDX_FP8_E4M3, w=W, k=K, sc=S, kd=D.IDX_MXFP4, n=4096, ks=KS, ke=KE,
             cand=CAND, cand_ld=4, nc=NC, block=128, rows=4, out=OUT, ld=512)
    a.update(kw)
    return L.idx_logits_sparse_blocks(a["q"], a["qd"], a["w"], a["k"], a["sc"], a["kd"], a["n"],
                                      a["ks"], a["ke"], a["cand"], a["cand_ld"], a["nc"], a["block"],
                                      a["rows"], a["out"], a["ld"], None)


def _paged_sparse(L, **kw):
    a = dict(q=Q, qd=D.IDX_FP8_E4M3, w=W, k=K, sc=S, kd=D.IDX_MXFP4, npages=100, page=128, bt=BT,
             bt_rows=4, bt_ld=16, sl=SL, rr=None, cand=CAND, cand_ld=4, nc=NC, block=128, rows=4, out=OUT, ld=512)
    a.update(kw)
    return L.idx_logits_paged_sparse_blocks(a["q"], a["qd"], a["w"], a["k"], a["sc"], a["kd"], a["npages"],
                                            a["page"], a["bt"], a["bt_rows"], a["bt_ld"], a["sl"], a["rr"],
                                            a["cand"], a["cand_ld"], a["nc"], a["block"], a["rows"], a["out"],
                                            a["ld"], None)


def _topk(L, **kw):
    a = dict(lg=OUT, ld=1024, lens=None, ncols=1024, rows=4, k=256, oi=Q, ov=None, old=256,
             flags=0, ws=None, wsb=0)
    a.update(kw)
    return L.idx_topk(a["lg"], a["ld"], a["lens"], a["ncols"], a["rows"], a["k"], a["oi"], a["ov"],
                      a["old"], a["flags"], a["ws"], a["wsb"], None)


ARG, UNS, WSP = D.IDX_ERR_ARG, D.IDX_ERR_UNSUPPORTED, D.IDX_ERR_WORKSPACE

CASES = [
    ("dense null q", _dense, dict(q=None), ARG),
    ("dense null w", _dense, dict(w=None), ARG),
    ("dense null out", _dense, dict(out=None), ARG),
    ("dense null scale", _dense, dict(sc=None), ARG),
    ("dense null ranges", _dense, dict(ks=None), ARG),
    ("dense negative rows", _dense, dict(rows=-1), ARG),
    ("dense negative n_keys", _dense, dict(n=-5), ARG),
    ("dense ld zero", _dense, dict(ld=0), ARG),
    ("dense ld too large", _dense, dict(ld=1 << 31), ARG),
    ("dense misaligned q", _dense, dict(q=Q + 8), ARG),
    ("dense misaligned k", _dense, dict(k=K + 4), ARG),
    ("dense misaligned w", _dense, dict(w=W + 2), ARG),
    ("dense w only 4-byte aligned", _dense, dict(w=W + 4), ARG),
    ("dense misaligned out", _dense, dict(out=OUT + 1), ARG),
    ("dense misaligned scale", _dense, dict(sc=S + 2), ARG),
    ("dense misaligned ranges", _dense, dict(ke=KE + 2), ARG),
    ("dense bf16 q fp8 k", _dense, dict(qd=D.IDX_BF16), UNS),
    ("dense fp8 q bf16 k", _dense, dict(kd=D.IDX_BF16), UNS),
    ("dense unknown dtype", _dense, dict(kd=9), UNS),
    ("paged page 32", _paged, dict(page=32), UNS),
    ("paged page 96", _paged, dict(page=96), UNS),
    ("paged bf16", _paged, dict(qd=D.IDX_BF16, kd=D.IDX_BF16), UNS),
    ("paged no pages", _paged, dict(npages=0), ARG),
    ("paged null table", _paged, dict(bt=None), ARG),
    ("paged null lens", _paged, dict(sl=None), ARG),
    ("paged bt_ld zero", _paged, dict(bt_ld=0), ARG),
    ("paged bt_ld too large", _paged, dict(bt_ld=1 << 25), ARG),
    ("paged bt_ld wrapping", _paged, dict(bt_ld=1 << 58), ARG),
    ("paged too few table rows", _paged, dict(bt_rows=3), ARG),
    ("paged misaligned row_req", _paged, dict(rr=SL + 2), ARG),
    ("sparse block 100", _sparse, dict(block=100), UNS),
    ("sparse bf16", _sparse, dict(qd=D.IDX_BF16, kd=D.IDX_BF16), UNS),
    ("sparse ld too small", _sparse, dict(ld=511), ARG),
    ("sparse null cand", _sparse, dict(cand=None), ARG),
    ("sparse null n_cols", _sparse, dict(nc=None), ARG),
    ("sparse cand_ld zero", _sparse, dict(cand_ld=0), ARG),
    ("sparse cand_ld wrapping", _sparse, dict(cand_ld=1 << 57, ld=1 << 40), ARG),
    ("paged sparse page not a multiple of the block", _paged_sparse, dict(page=192), UNS),
    ("paged sparse page smaller than the block", _paged_sparse, dict(page=64), UNS),
    ("paged sparse page 96", _paged_sparse, dict(page=96, block=64), UNS),
    ("paged sparse block 100", _paged_sparse, dict(block=100), UNS),
    ("paged sparse bf16", _paged_sparse, dict(qd=D.IDX_BF16, kd=D.IDX_BF16), UNS),
    ("paged sparse ld too small", _paged_sparse, dict(ld=511), ARG),
    ("paged sparse null table", _paged_sparse, dict(bt=None), ARG),
    ("paged sparse null cand", _paged_sparse, dict(cand=None), ARG),
    ("paged sparse null n_cols", _paged_sparse, dict(nc=None), ARG),
    ("paged sparse no pages", _paged_sparse, dict(npages=0), ARG),
    ("paged sparse too few table rows", _paged_sparse, dict(bt_rows=3), ARG),
    ("paged sparse misaligned cand", _paged_sparse, dict(cand=CAND + 2), ARG),
    ("paged sparse cand_ld zero", _paged_sparse, dict(cand_ld=0), ARG),
    ("topk k zero", _topk, dict(k=0), UNS),
    ("topk k too large", _topk, dict(k=2049, old=4096), UNS),
    ("topk out_ld < k", _topk, dict(old=255), ARG),
    ("topk ld < n_cols", _topk, dict(ncols=2048), ARG),
    ("topk null logits", _topk, dict(lg=None), ARG),
    ("topk null out", _topk, dict(oi=None), ARG),
    ("topk misaligned lens", _topk, dict(lens=KS + 1), ARG),
    ("topk bad flags", _topk, dict(flags=6), ARG),
    ("topk long rows without workspace", _topk, dict(ld=131072, ncols=131072), WSP),
    ("topk long rows small workspace", _topk, dict(ld=131072, ncols=131072, ws=WS, wsb=4096), WSP),
    ("topk long rows misaligned workspace", _topk, dict(ld=131072, ncols=131072, ws=WS + 8, wsb=1 << 30), ARG),
    ("topk negative rows", _topk, dict(rows=-2), ARG),
]


@pytest.mark.parametrize("name,fn,kw,status", CASES, ids=[c[0] for c in CASES])
def test_host_rejects(L, name, fn, kw, status):
    got = fn(L, **kw)
    assert got == status, f"{name}: got {got}, last error {L.idx_last_error()!r}"
    assert L.idx_last_error(), "a failed call must set idx_last_error"


def test_paged_sparse_accepts_pages_that_are_block_multiples(L):
    """page_size a multiple of block_size passes the host checks (the call is only checked
    here: zero rows)."""
    for page, block in ((64, 64), (128, 64), (128, 128), (256, 128), (512, 256)):
        assert _paged_sparse(L, page=page, block=block, rows=0) == D.IDX_OK


@pytest.mark.parametrize("fn", [_dense, _paged, _sparse, _paged_sparse, _topk])
def test_zero_rows_is_noop(L, fn):
    assert fn(L, rows=0) == D.IDX_OK
    assert L.idx_last_error() == b""


def _problem(**kw):
    a = dict(mode=D.IDX_MODE_DENSE, rows=4, q=Q, q_dtype=D.IDX_FP8_E4M3, k_dtype=D.IDX_FP8_E4M3,
             w=W, k=K, k_scale=S, n_keys=4096, row_ks=KS, row_ke=KE, max_cols=4096)
    a.update(kw)
    return D.idx_problem(**a)


def _r256(x):
    return (x + 255) // 256 * 256


def _select_layouts(L, rows, width):
    """Workspace of the two idx_select layouts the header describes: the one-pass selection
    (1024 workgroups x 2 histogram slots of 2048 + 256 words, a counter per row, rows + 1
    step offsets, a 16-byte segment record per 64-column step, 64 keys of 8 bytes per step,
    spill score rows) and scores then top-k (score rows, scored lengths, the top-k
    workspace); ldw = width rounded up to 64."""
    ldw = (width + 63) // 64 * 64
    steps = rows * (ldw // 64)
    one = sum(_r256(b) for b in (1024 * 2 * 2304 * 4, rows * 8, (rows + 1) * 8, steps * 16, steps * 64 * 8,
                                  rows * ldw * 4))
    two = _r256(rows * ldw * 4) + _r256(rows * 4) + L.idx_topk_workspace(rows, width, 2048)
    return one, two


def test_select_workspace_sizes(L):
    # fewer than 8 rows: scores then top-k only
    p = _problem(max_cols=4000)
    _, two = _select_layouts(L, 4, 4000)
    assert L.idx_select_workspace(C.byref(p), 2048) == two
    p = _problem(rows=16, max_cols=4000)
    one, two = _select_layouts(L, 16, 4000)
    assert L.idx_select_workspace(C.byref(p), 2048) == max(one, two)
    p = _problem(rows=64, mode=D.IDX_MODE_PAGED, page_size=64, block_table=BT, bt_rows=64, bt_ld=2048,
                 seq_lens=SL)
    one, two = _select_layouts(L, 64, 131072)
    assert L.idx_select_workspace(C.byref(p), 2048) == max(one, two)
    p = _problem(rows=64, mode=D.IDX_MODE_SPARSE_BLOCKS, k_dtype=D.IDX_MXFP4, cand_blocks=CAND, cand_ld=64,
                 n_cols=NC, block_size=128)
    one, two = _select_layouts(L, 64, 8192)
    assert L.idx_select_workspace(C.byref(p), 2048) == max(one, two)
    # a prefill chunk (IDX_MODE_PREFILL, fp8, >= 256 rows) takes the tiled kernel and the
    # two-pass layout; the same rows as dense decode rows can take the one-pass selection
    p = _problem(rows=300, max_cols=5000, mode=D.IDX_MODE_PREFILL)
    one, two = _select_layouts(L, 300, 5000)
    assert L.idx_select_workspace(C.byref(p), 2048) == two
    p = _problem(rows=300, max_cols=5000)
    assert L.idx_select_workspace(C.byref(p), 2048) == max(one, two)
    # a small prefill chunk (fewer than 256 rows) runs the scan like dense rows
    p = _problem(rows=100, max_cols=5000, mode=D.IDX_MODE_PREFILL)
    one, two = _select_layouts(L, 100, 5000)
    assert L.idx_select_workspace(C.byref(p), 2048) == max(one, two)


SELECT_CASES = [
    ("null problem", None, dict(), ARG),
    ("workspace missing", _problem(), dict(ws=None, wsb=0), WSP),
    ("workspace small", _problem(), dict(wsb=1000), WSP),
    ("workspace misaligned", _problem(), dict(ws=WS + 16), ARG),
    ("k zero", _problem(), dict(k=0), UNS),
    ("k too large", _problem(), dict(k=4096, old=4096), UNS),
    ("out_ld < k", _problem(), dict(old=100), ARG),
    ("dense max_cols zero", _problem(max_cols=0), dict(), ARG),
    ("unknown mode", _problem(mode=7), dict(), ARG),
    ("unknown flag", _problem(), dict(flags=8), ARG),
    ("paged page 16", _problem(mode=D.IDX_MODE_PAGED, page_size=16, block_table=BT, bt_rows=4,
                                bt_ld=4, seq_lens=SL), dict(), UNS),
    ("paged table rows", _problem(mode=D.IDX_MODE_PAGED, page_size=64, block_table=BT, bt_rows=2,
                                   bt_ld=4, seq_lens=SL), dict(), ARG),
    ("sparse dtype", _problem(mode=D.IDX_MODE_SPARSE_BLOCKS, q_dtype=D.IDX_BF16,
                              k_dtype=D.IDX_BF16, cand_blocks=CAND, cand_ld=4, n_cols=NC,
                              block_size=128), dict(), UNS),
]


@pytest.mark.parametrize("name,p,kw,status", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_rejects(L, name, p, kw, status):
    a = dict(k=256, oi=OUT, ov=None, old=256, flags=0, ws=WS, wsb=1 << 30)
    a.update(kw)
    got = L.idx_select(None if p is None else C.byref(p), a["k"], a["oi"], a["ov"], a["old"],
                       a["flags"], a["ws"], a["wsb"], None)
    assert got == status, f"{name}: got {got}, last error {L.idx_last_error()!r}"


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(D, "_LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(D, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        D.lib()


def test_read_probe_rejects_bad_arguments(L):
    """The bandwidth probe checks its arguments on the host before anything is enqueued."""
    assert L.idx_read_probe(None, 1024, C.c_void_p(0x1000), None) == D.IDX_ERR_ARG
    assert L.idx_read_probe(C.c_void_p(0x1000), 1024, None, None) == D.IDX_ERR_ARG
    assert L.idx_read_probe(C.c_void_p(0x1008), 1024, C.c_void_p(0x2000), None) == D.IDX_ERR_ARG  # misaligned
    assert L.idx_read_probe(C.c_void_p(0x1000), 1000, C.c_void_p(0x2000), None) == D.IDX_ERR_ARG  # not a multiple of 16
    assert b"idx_read_probe" in L.idx_last_error()


def test_kcache_write_rejects_bad_arguments(L):
    """The key-cache writer checks its arguments on the host before anything is enqueued."""
    ok = dict(k=C.c_void_p(0x1000), nd=D.IDX_BF16, n=4, s=C.c_void_p(0x2000), c=C.c_void_p(0x3000),
              sc=C.c_void_p(0x4000), kd=D.IDX_FP8_E4M3, ns=64)

    def call(**kw):
        a = {**ok, **kw}
        return L.idx_kcache_write(a["k"], a["nd"], a["n"], a["s"], a["c"], a["sc"], a["kd"], a["ns"], None)

    assert call(nd=D.IDX_FP8_E4M3) == D.IDX_ERR_UNSUPPORTED     # new keys must be bf16
    assert call(kd=D.IDX_BF16) == D.IDX_ERR_UNSUPPORTED         # cache must be fp8 or MXFP4
    assert call(n=-1) == D.IDX_ERR_ARG
    assert call(ns=-5) == D.IDX_ERR_ARG
    assert call(s=None) == D.IDX_ERR_ARG
    assert call(c=C.c_void_p(0x3004)) == D.IDX_ERR_ARG        # cache not 16-byte aligned
    assert call(k=C.c_void_p(0x1008)) == D.IDX_ERR_ARG        # keys not 16-byte aligned
    assert call(n=0, s=None, c=None) == D.IDX_OK              # nothing to write
    assert b"idx_kcache_write" in L.idx_last_error() or L.idx_last_error() == b""


def test_candidate_blocks_rejects_bad_arguments(L):
    """The candidate-block publisher checks its arguments on the host before anything is
    enqueued."""
    ok = dict(lg=C.c_void_p(0x1000), ld=4096, lens=None, n=4096, rows=8, bs=128, top=16, c=C.c_void_p(0x2000),
              cld=16, nc=C.c_void_p(0x3000), ws=C.c_void_p(0x10000), wsb=1 << 20)

    def call(**kw):
        a = {**ok, **kw}
        return L.idx_candidate_blocks(a["lg"], a["ld"], a["lens"], a["n"], a["rows"], a["bs"], a["top"], a["c"],
                                      a["cld"], a["nc"], a["ws"], a["wsb"], None)

    assert L.idx_candidate_blocks_workspace(8, 4096) == 8 * 64 * 4
    assert L.idx_candidate_blocks_workspace(3, 65) == 256  # 2 pieces per row, rounded to 4
    assert L.idx_candidate_blocks_workspace(8, 0) == 0
    assert call(bs=100) == D.IDX_ERR_UNSUPPORTED           # not a multiple of 64
    assert call(bs=8192) == D.IDX_ERR_UNSUPPORTED          # above 4096
    assert call(n=64 * 16385, ld=64 * 16385, bs=64) == D.IDX_ERR_UNSUPPORTED  # more than 16384 blocks
    assert call(top=0) == D.IDX_ERR_ARG
    assert call(top=17) == D.IDX_ERR_ARG                    # cand_ld < n_top
    assert call(ld=4095) == D.IDX_ERR_ARG                   # ld < n_cols
    assert call(rows=-1) == D.IDX_ERR_ARG
    assert call(lg=None) == D.IDX_ERR_ARG
    assert call(nc=None) == D.IDX_ERR_ARG
    assert call(c=C.c_void_p(0x2002)) == D.IDX_ERR_ARG       # misaligned
    assert call(ws=None) == D.IDX_ERR_WORKSPACE
    assert call(wsb=100) == D.IDX_ERR_WORKSPACE
    assert call(ws=C.c_void_p(0x10010)) == D.IDX_ERR_ARG     # workspace not 256-byte aligned
    assert call(rows=0, lg=None, c=None, nc=None) == D.IDX_OK
    assert b"idx_candidate_blocks" in L.idx_last_error() or L.idx_last_error() == b""


def test_python_binding_rejects_host_tensors():
    """The kernels take device pointers: host tensors are refused before any call."""
    import torch
    q = torch.zeros((2, 64, 128), dtype=torch.uint8)
    w = torch.zeros((2, 64), dtype=torch.float32)
    k = torch.zeros((256, 128), dtype=torch.uint8)
    sc = torch.ones(256, dtype=torch.float32)
    ks = torch.zeros(2, dtype=torch.int32)
    ke = torch.full((2,), 256, dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        D.idx_logits(q, w, k, sc, ks, ke, k_dtype="fp8", ld=256)
    with pytest.raises(ValueError, match="device tensor"):
        D.dense_problem(q, w, k, sc, ks, ke, k_dtype="fp8", max_cols=256)
    with pytest.raises(ValueError, match="device tensor"):
        D.idx_topk(torch.zeros((2, 256), dtype=torch.float32), 8)
    with pytest.raises(ValueError, match="device tensor"):
        D.idx_read_probe(torch.zeros(16, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="k_dtype"):
        D.idx_logits(q, w, k, sc, ks, ke, k_dtype="fp16", ld=256)
