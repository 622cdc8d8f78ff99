"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle (the ``oracle`` module,
possibly running a planted-mistake build through ``oracle.variant``) disagrees with
something the pages or the mathematics fix:

* decode tables against torch's independent fp8 / bf16 casts and the OCP spec values
  (golden files),
* Eq. (1) against an exact rational brute force (``fractions.Fraction``, decoding through
  torch / the golden e2m1 table, one correct RNE rounding to fp32),
* special cases that reduce Eq. (1) to a numpy matrix product,
* invariants (key / head permutation, linearity in w, power-of-two scale homogeneity,
  non-negativity, masking),
* top-k against the worked example in the golden file and against numpy's lexsort,
* the equivalences between the three ways of naming keys (paged vs contiguous,
  candidate blocks vs dense-masked).

Sizes are tiny so that the whole list runs in seconds.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import oracle as O
import synth

GOLDEN = Path(__file__).resolve().parent / "golden"


# ----------------------------------------------------------------------------- helpers


def _golden_lines(name):
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if line and not line.startswith("#"):
            yield line.split()


def e2m1_golden() -> dict[int, float]:
    return {int(a): float(b) for a, b in _golden_lines("ocp_e2m1.txt")}


def torch_fp8(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_bf16(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def frac_to_f32(x: Fraction) -> np.float32:
    """Exact rational -> float32 with one round-to-nearest-even (normal and subnormal)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = max(e, -126) - 23
    m = a / Fraction(2) ** quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** quantum))


def near_f32_tie(x: Fraction) -> bool:
    """True when x lies within 2^-40 (relative) of a float32 rounding midpoint, where an
    fp64 evaluation may legitimately round to either neighbour."""
    if x == 0:
        return False
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    frac = (a / quantum) % 1
    return abs(frac - Fraction(1, 2)) * quantum < a * Fraction(1, 2 ** 40)


def exact_scores(qv, wv, kv):
    """Eq. (1) in exact rationals: qv [H][D], wv [H], kv [N][D] of Fractions -> [N]."""
    out = []
    for key in kv:
        acc = Fraction(0)
        for j in range(len(qv)):
            dot = sum((a * b for a, b in zip(qv[j], key)), Fraction(0))
            acc += wv[j] * (dot if dot > 0 else Fraction(0))
        out.append(acc)
    return out


def _fr(arr):
    return [[Fraction(float(v)) for v in row] for row in np.asarray(arr, dtype=np.float64)]


def _dense_one(q, qd, w, k, sc, kd, n):
    return O.logits_dense(q[None], qd, w[None], k, sc, kd, np.array([0], np.int32),
                          np.array([n], np.int32))[0]


def _check_exact(got, exact, what):
    for i, (g, x) in enumerate(zip(got, exact)):
        want = frac_to_f32(x)
        if not (g == want or near_f32_tie(x)):
            raise AssertionError(f"{what}: key {i}: oracle {g!r} exact {want!r} ({float(x)!r})")


# ----------------------------------------------------------------------------- decoding


def pin_fp8_table_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = O.decode_fp8(codes), torch_fp8(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref)), "fp8 NaN codes differ from torch"
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok]), "fp8 values differ from torch"
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok])), "fp8 zero signs differ"


def pin_fp8_spec_values():
    for code, val in _golden_lines("ocp_fp8_e4m3fn_special.txt"):
        got = float(O.decode_fp8([int(code, 16)])[0])
        want = float(val)
        if np.isnan(want):
            assert np.isnan(got), f"fp8 {code} should be NaN"
        else:
            assert got == want and np.signbit(got) == np.signbit(want), f"fp8 {code}: {got} != {want}"


def pin_e2m1_spec_table():
    table = e2m1_golden()
    got = O.decode_e2m1(np.arange(16))
    for c in range(16):
        assert got[c] == table[c] and np.signbit(got[c]) == np.signbit(table[c]), f"e2m1 code {c}"


def pin_ue8m0_closed_form():
    got = O.decode_ue8m0(np.arange(256))
    for e in range(255):
        assert got[e] == float(Fraction(2) ** (e - 127)), f"ue8m0 {e}"
    assert np.isnan(got[255]), "ue8m0 255 must be NaN"


def pin_bf16_vs_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=2000, dtype=np.uint32).astype(np.uint16)
    ours, ref = O.decode_bf16(bits), torch_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ----------------------------------------------------------------------------- Eq. (1) exact


def pin_bruteforce_fp8():
    rng = np.random.default_rng(11)
    for heads, dim, n in [(1, 4, 9), (2, 4, 9), (4, 32, 7), (64, 128, 4)]:
        q = synth.to_fp8_e4m3fn(rng.standard_normal((heads, dim)).astype(np.float32) * 2)
        k = synth.to_fp8_e4m3fn(rng.standard_normal((n, dim)).astype(np.float32) * 2)
        sc = rng.uniform(0.5, 2.0, n).astype(np.float32)
        w = (rng.standard_normal(heads) / 8).astype(np.float32)
        got = _dense_one(q, "fp8", w, k, sc, "fp8", n)
        kv = [[Fraction(float(v)) * Fraction(float(sc[i])) for v in row]
              for i, row in enumerate(torch_fp8(k))]
        exact = exact_scores(_fr(torch_fp8(q)), [Fraction(float(x)) for x in w], kv)
        _check_exact(got, exact, f"fp8 H={heads} D={dim}")


def pin_bruteforce_bf16():
    rng = np.random.default_rng(12)
    for heads, dim, n in [(1, 4, 9), (2, 4, 9), (64, 128, 3)]:
        q = synth.to_bf16_bits(rng.standard_normal((heads, dim)).astype(np.float32) / 11)
        k = synth.to_bf16_bits(rng.standard_normal((n, dim)).astype(np.float32) / 11)
        w = (rng.standard_normal(heads) / 8).astype(np.float32)
        got = _dense_one(q, "bf16", w, k, None, "bf16", n)
        exact = exact_scores(_fr(torch_bf16(q)), [Fraction(float(x)) for x in w],
                             _fr(torch_bf16(k)))
        _check_exact(got, exact, f"bf16 H={heads} D={dim}")


def _mx_decode_golden(codes, scales, dim):
    table = e2m1_golden()
    out = []
    for row_c, row_s in zip(codes, scales):
        vals = []
        for i in range(dim):
            byte = int(row_c[i // 2])
            nib = byte & 0xF if i % 2 == 0 else byte >> 4
            vals.append(Fraction(table[nib]) * Fraction(2) ** (int(row_s[i // 32]) - 127))
        out.append(vals)
    return out


def pin_bruteforce_mxfp4():
    rng = np.random.default_rng(13)
    for heads, dim, n in [(1, 32, 9), (2, 64, 7), (64, 128, 4)]:
        q = synth.to_fp8_e4m3fn(rng.standard_normal((heads, dim)).astype(np.float32) * 2)
        codes, scales = synth.to_mxfp4(rng.standard_normal((n, dim)) * rng.uniform(0.1, 10, (n, 1)))
        w = (rng.standard_normal(heads) / 8).astype(np.float32)
        got = _dense_one(q, "fp8", w, codes, scales, "mxfp4", n)
        exact = exact_scores(_fr(torch_fp8(q)), [Fraction(float(x)) for x in w],
                             _mx_decode_golden(codes, scales, dim))
        _check_exact(got, exact, f"mxfp4 H={heads} D={dim}")


# ----------------------------------------------------------------------------- special cases


def pin_single_head_is_relu_matmul():
    """H = 1, w = 1: I = ReLU(q . k), i.e. np.maximum(K @ q, 0)."""
    rng = np.random.default_rng(21)
    n = 300
    q = synth.to_fp8_e4m3fn(rng.standard_normal((1, 128)).astype(np.float32))
    k = synth.to_fp8_e4m3fn(rng.standard_normal((n, 128)).astype(np.float32))
    sc = rng.uniform(0.5, 2.0, n).astype(np.float32)
    got = _dense_one(q, "fp8", np.ones(1, np.float32), k, sc, "fp8", n)
    ref = np.maximum((torch_fp8(k) * sc[:, None].astype(np.float64)) @ torch_fp8(q)[0], 0.0)
    assert np.allclose(got, ref, rtol=2e-7, atol=0), "H=1 ReLU(q.k) mismatch"
    assert (got == 0).sum() > n // 4, "expected many ReLU zeros"


def pin_positive_inputs_are_matvec():
    """All-positive q and keys, w = 1: ReLU is inactive and I = (sum_j q_j) . k."""
    rng = np.random.default_rng(22)
    n, heads = 200, 64
    q = synth.to_fp8_e4m3fn(np.abs(rng.standard_normal((heads, 128))).astype(np.float32))
    k = synth.to_fp8_e4m3fn(np.abs(rng.standard_normal((n, 128))).astype(np.float32))
    got = _dense_one(q, "fp8", np.ones(heads, np.float32), k, np.ones(n, np.float32), "fp8", n)
    ref = torch_fp8(k) @ torch_fp8(q).sum(axis=0)
    assert np.allclose(got, ref, rtol=2e-7, atol=0), "positive matvec mismatch"


def pin_zero_weights():
    """w = 0 gives I = 0 everywhere, so the top-k is the first k keys (lower index wins)."""
    case = synth.batched_decode(seed=31, rows=2, n=300, topk=17)
    case.w = np.zeros_like(case.w)
    idx, val = O.select_case(case)
    assert np.all(val == 0)
    assert np.array_equal(idx, np.tile(np.arange(17, dtype=np.int32), (2, 1)))


def pin_nonnegative_for_nonnegative_w():
    case = synth.batched_decode(seed=32, rows=3, n=400, topk=8)
    case.w = np.abs(case.w)
    lg = O.logits_dense(case.q, case.q_dtype, case.w, case.k, case.k_scale, case.k_dtype,
                        case.row_ks, case.row_ke)
    assert np.all(lg >= 0) and np.any(lg > 0)


# ----------------------------------------------------------------------------- invariants


def pin_key_permutation():
    """Permuting the keys permutes the logits and maps the selected indices through the
    permutation (the selection must use the actual indices, not the first k)."""
    rng = np.random.default_rng(41)
    case = synth.batched_decode(seed=41, rows=1, n=500, topk=20)
    perm = rng.permutation(500)
    base = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale, "fp8", case.row_ks, case.row_ke)
    pl = O.logits_dense(case.q, "fp8", case.w, case.k[perm], case.k_scale[perm], "fp8",
                        case.row_ks, case.row_ke)
    assert np.array_equal(pl[0], base[0][perm]), "logits not permutation-equivariant"
    i0, _ = O.topk(base, 20)
    i1, _ = O.topk(pl, 20)
    assert np.unique(base[0]).size == 500
    assert np.array_equal(perm[i1[0]], i0[0]), "top-k not permutation-equivariant"


def pin_head_permutation():
    rng = np.random.default_rng(42)
    case = synth.batched_decode(seed=42, rows=2, n=300, topk=8)
    perm = rng.permutation(64)
    a = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale, "fp8", case.row_ks, case.row_ke)
    b = O.logits_dense(case.q[:, perm], "fp8", case.w[:, perm], case.k, case.k_scale, "fp8",
                       case.row_ks, case.row_ke)
    assert np.allclose(a, b, rtol=1.2e-7, atol=0), "head order changed the score"


def pin_linear_in_w():
    case = synth.batched_decode(seed=43, rows=2, n=300, topk=8)
    args = (case.k, case.k_scale, "fp8", case.row_ks, case.row_ke)
    a = O.logits_dense(case.q, "fp8", case.w, *args)
    b = O.logits_dense(case.q, "fp8", case.w * 2, *args)
    assert np.array_equal(b, a * 2), "scaling w by 2 must scale I by 2 exactly"
    w2 = np.random.default_rng(43).standard_normal(case.w.shape).astype(np.float32) / 8
    c = O.logits_dense(case.q, "fp8", w2, *args)
    d = O.logits_dense(case.q, "fp8", case.w + w2, *args)
    assert np.allclose(d, a.astype(np.float64) + c, rtol=1e-5, atol=1e-5), "I not additive in w"


def pin_scale_homogeneity():
    """Multiplying a token's fp8 scale by 4 (or its UE8M0 exponents by +2) multiplies
    its score by 4 exactly."""
    case = synth.batched_decode(seed=44, rows=2, n=300, topk=8)
    a = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale, "fp8", case.row_ks, case.row_ke)
    b = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale * 4, "fp8", case.row_ks, case.row_ke)
    assert np.array_equal(b, a * 4)
    sp = synth.sparse_blocks(seed=45, rows=2, ctx=1024, n_blocks=3, block=128, topk=8,
                             poison_noncand=False)
    args = (sp.row_ks, sp.row_ke, sp.cand, sp.n_cols, sp.block)
    a = O.logits_sparse(sp.q, "fp8", sp.w, sp.k, sp.k_scale, "mxfp4", *args)
    b = O.logits_sparse(sp.q, "fp8", sp.w, sp.k, sp.k_scale + 2, "mxfp4", *args)
    fin = np.isfinite(a)
    assert np.array_equal(b[fin], a[fin] * 4)


def pin_scale_per_group():
    """Each UE8M0 byte scales only its own 32 elements: raising group g's exponent by one
    equals doubling q's dims 32g..32g+31 (fp8 doubling is exact away from the top binade)."""
    sp = synth.sparse_blocks(seed=46, rows=2, ctx=512, n_blocks=2, block=128, topk=8,
                             poison_noncand=False)
    args = (sp.row_ks, sp.row_ke, sp.cand, sp.n_cols, sp.block)
    qf = torch_fp8(sp.q)
    for g in range(4):
        sc = sp.k_scale.copy()
        sc[:, g] += 1
        a = O.logits_sparse(sp.q, "fp8", sp.w, sp.k, sc, "mxfp4", *args)
        q2f = qf.copy()
        q2f[:, :, 32 * g:32 * g + 32] *= 2
        q2 = synth.to_fp8_e4m3fn(q2f.astype(np.float32))
        assert np.array_equal(torch_fp8(q2), q2f), "doubling must stay exact"
        b = O.logits_sparse(q2, "fp8", sp.w, sp.k, sp.k_scale, "mxfp4", *args)
        assert np.array_equal(a, b), f"group {g} scale does not match its 32 dims"


def pin_masking():
    """Keys outside a row's range are never read: poisoned (NaN) neighbours do not leak,
    and columns past the row's length are -inf."""
    case = synth.batched_decode(seed=47, rows=4, n=200, topk=8, ragged=True, gap=37)
    lg = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale, "fp8", case.row_ks,
                        case.row_ke, ld=260)
    for r in range(4):
        L = int(case.row_ke[r] - case.row_ks[r])
        assert np.all(np.isfinite(lg[r, :L])), "poison leaked into a valid key"
        assert np.all(lg[r, L:] == -np.inf)


# ----------------------------------------------------------------------------- top-k


def pin_topk_worked_example():
    lines = {ln[0]: ln[1:] for ln in _golden_lines("topk_worked_example.txt")}
    scores = np.array([[float(x) for x in lines["scores"]]], np.float32)
    k = int(lines["k"][0])
    want = np.array([[int(x) for x in lines["selected"]]], np.int32)
    idx, val = O.topk(scores, k)
    assert np.array_equal(idx, want), f"worked example: {idx} != {want}"
    assert np.array_equal(val, scores[0][want[0]][None])


def pin_topk_vs_lexsort():
    """top-k = prefix of the full (value desc, index asc) order, over rows with many ties,
    signed zeros and absent (-inf / NaN) entries."""
    rng = np.random.default_rng(51)
    rows, n, k = 6, 700, 50
    lg = rng.integers(-20, 20, size=(rows, n)).astype(np.float32) / 4
    lg[rng.random((rows, n)) < 0.05] = -0.0
    lg[rng.random((rows, n)) < 0.1] = -np.inf
    lg[rng.random((rows, n)) < 0.02] = np.nan
    lg[2] = np.where(rng.random(n) < 0.5, 0.0, -0.0)
    lg[3, :] = -np.inf
    lg[3, :10] = 1.0
    lens = np.array([n, n - 1, 333, n, 17, 0], np.int32)
    idx, val = O.topk(lg, k, lens)
    for r in range(rows):
        cols = np.arange(lens[r])
        v = lg[r, :lens[r]].astype(np.float64)
        ok = np.isfinite(v) | (v == np.inf)
        cols, v = cols[ok], v[ok]
        v = np.where(v == 0, 0.0, v)
        order = cols[np.lexsort((cols, -v))][:k]
        want = np.full(k, -1, np.int32)
        want[:order.size] = order
        assert np.array_equal(idx[r], want), f"row {r}: top-k is not the sort prefix"
        assert np.array_equal(val[r][:order.size], lg[r][order])
        assert np.all(val[r][order.size:] == -np.inf)


def pin_topk_all_equal():
    lg = np.full((2, 100), 3.5, np.float32)
    idx, _ = O.topk(lg, 30)
    assert np.array_equal(idx, np.tile(np.arange(30, dtype=np.int32), (2, 1)))


def pin_topk_pads_short_rows():
    lg = np.array([[1.0, 5.0, -np.inf, 2.0]], np.float32)
    idx, val = O.topk(lg, 6)
    assert idx.tolist() == [[1, 3, 0, -1, -1, -1]]
    assert val[0, :3].tolist() == [5.0, 2.0, 1.0] and np.all(val[0, 3:] == -np.inf)


# ----------------------------------------------------------------------------- candidate blocks


def pin_candidate_blocks_by_hand():
    """Blocks of 4: scores [.1 .5 -1 2 | 3 0 0 0 | 1 1 1 1 | -inf x4 | 3 -inf nan 2].
    Block maxima 2, 3, 1, (none), 3: the best two are blocks 1 and 4 (equal 3, lower id
    first), published ascending; with n_top = 4 block 0 joins, block 3 never does."""
    lg = np.array([[0.1, 0.5, -1, 2, 3, 0, 0, 0, 1, 1, 1, 1, -np.inf, -np.inf, -np.inf, -np.inf,
                    3, -np.inf, np.nan, 2]], np.float32)
    cand, n = O.candidate_blocks(lg, 4, 2)
    assert cand.tolist() == [[1, 4]] and n.tolist() == [2]
    cand, n = O.candidate_blocks(lg, 4, 3)
    assert cand.tolist() == [[0, 1, 4]] and n.tolist() == [3]
    cand, n = O.candidate_blocks(lg, 4, 6)
    assert cand.tolist() == [[0, 1, 2, 4, -1, -1]] and n.tolist() == [4]
    # the last block may be partial: lens 17 keeps token 16 (score 3) of block 4
    cand, n = O.candidate_blocks(lg, 4, 1, lens=np.array([17], np.int32))
    assert cand.tolist() == [[1]] and n.tolist() == [1]
    cand, n = O.candidate_blocks(lg, 4, 2, lens=np.array([16], np.int32))
    assert cand.tolist() == [[0, 1]] and n.tolist() == [2]


def pin_candidate_blocks_vs_token_ranking():
    """The n_top best blocks by maximum are the first n_top distinct blocks met walking
    the row's tokens in the exact top-k order (value desc, index asc): a block's rank is
    that of its best token, and equal maxima order by the lower token, hence the lower
    block. Checked by that walk over rows with ties, signed zeros, absent entries and
    ragged lengths."""
    rng = np.random.default_rng(53)
    rows, n = 7, 900
    lg = rng.integers(-12, 12, size=(rows, n)).astype(np.float32) / 4
    lg[rng.random((rows, n)) < 0.05] = -0.0
    lg[rng.random((rows, n)) < 0.2] = -np.inf
    lg[rng.random((rows, n)) < 0.02] = np.nan
    lg[4, 128:512] = -np.inf
    lg[5] = 1.5
    lens = np.array([n, n - 5, 640, 129, n, 300, 0], np.int32)
    for block, n_top in ((64, 5), (128, 3), (128, 8), (256, 2)):
        cand, n_cand = O.candidate_blocks(lg, block, n_top, lens)
        for r in range(rows):
            cols = np.arange(lens[r])
            v = lg[r, :lens[r]].astype(np.float64)
            ok = ~np.isnan(v) & (v != -np.inf)
            cols, v = cols[ok], np.where(v[ok] == 0, 0.0, v[ok])
            seen = []
            for c in cols[np.lexsort((cols, -v))]:
                if int(c) // block not in seen:
                    seen.append(int(c) // block)
                if len(seen) == n_top:
                    break
            want = sorted(seen) + [-1] * (n_top - len(seen))
            assert cand[r].tolist() == want, f"row {r} block {block}: {cand[r]} != {want}"
            assert n_cand[r] == len(seen)


def pin_candidate_blocks_all_equal():
    lg = np.full((2, 1000), -2.25, np.float32)
    cand, n = O.candidate_blocks(lg, 128, 3)
    assert cand.tolist() == [[0, 1, 2]] * 2 and n.tolist() == [3, 3]
    cand, n = O.candidate_blocks(lg, 128, 10)
    assert cand.tolist() == [list(range(8)) + [-1, -1]] * 2 and n.tolist() == [8, 8]


# ----------------------------------------------------------------------------- key sources


def _paged_from_dense(case, page, perm_pages, rng):
    n = int(case.row_ke[0] - case.row_ks[0])
    rows = case.rows
    npg = (n + page - 1) // page
    P = rows * npg
    kp = np.full((P, page, 128), synth.FP8_NAN, np.uint8)
    sp = np.full((P, page), np.nan, np.float32)
    phys = rng.permutation(P) if perm_pages else np.arange(P)
    bt = np.full((rows, npg + 2), -1, np.int32)
    for r in range(rows):
        for p in range(npg):
            pid = int(phys[r * npg + p])
            bt[r, p] = pid
            lo = int(case.row_ks[r]) + p * page
            hi = min(lo + page, int(case.row_ke[r]))
            kp[pid, :hi - lo] = case.k[lo:hi]
            sp[pid, :hi - lo] = case.k_scale[lo:hi]
    return kp, sp, bt


def pin_paged_equals_contiguous():
    rng = np.random.default_rng(61)
    case = synth.batched_decode(seed=61, rows=3, n=333, topk=16)
    dense = O.logits_dense(case.q, "fp8", case.w, case.k, case.k_scale, "fp8", case.row_ks,
                           case.row_ke, ld=64 * 8)
    for perm in (False, True):
        kp, sp, bt = _paged_from_dense(case, 64, perm, rng)
        lens = (case.row_ke - case.row_ks).astype(np.int32)
        pg = O.logits_paged(case.q, "fp8", case.w, kp, sp, "fp8", bt, lens, ld=64 * 8)
        assert np.array_equal(pg, dense), f"paged (permuted={perm}) != contiguous"
    rr = np.array([2, 0, 1], np.int32)
    kp, sp, bt = _paged_from_dense(case, 64, True, rng)
    pg = O.logits_paged(case.q, "fp8", case.w, kp, sp, "fp8", bt[rr], lens, row_req=np.argsort(rr).astype(np.int32), ld=64 * 8)
    assert np.array_equal(pg, dense), "row -> request map not honoured"


def pin_sparse_equals_dense_masked():
    """Scoring only the candidate blocks and selecting over their columns gives exactly the
    selection of the dense route that scores every token and masks non-candidates."""
    for kd, seed in (("mxfp4", 71), ("fp8", 72)):
        sp = synth.sparse_blocks(seed=seed, rows=4, ctx=2048, n_blocks=5, block=128, topk=100,
                                 kdtype=kd, ragged=True, poison_noncand=False)
        idx_sparse, val_sparse = O.select_case(sp)
        dense = O.logits_dense(sp.q, "fp8", sp.w, sp.k, sp.k_scale, kd, sp.row_ks, sp.row_ke)
        mask = np.zeros_like(dense, dtype=bool)
        for r in range(sp.rows):
            for c in range(int(sp.n_cols[r])):
                tok = int(sp.cand[r, c // 128]) * 128 + c % 128
                if tok < dense.shape[1]:
                    mask[r, tok] = True
        masked = np.where(mask, dense, -np.inf).astype(np.float32)
        idx_dense, val_dense = O.topk(masked, 100)
        assert np.array_equal(idx_sparse, idx_dense), f"{kd}: sparse != dense-masked"
        assert np.array_equal(val_sparse, val_dense)


def pin_sparse_columns():
    sp = synth.sparse_blocks(seed=73, rows=3, ctx=1000, n_blocks=4, block=128, topk=10,
                             kdtype="fp8", ragged=True, poison_noncand=False)
    lg = O.logits_sparse(sp.q, "fp8", sp.w, sp.k, sp.k_scale, "fp8", sp.row_ks, sp.row_ke,
                         sp.cand, sp.n_cols, sp.block)
    dense = O.logits_dense(sp.q, "fp8", sp.w, sp.k, sp.k_scale, "fp8", sp.row_ks, sp.row_ke,
                           ld=1024)
    for r in range(3):
        for c in range(lg.shape[1]):
            tok = int(sp.cand[r, c // 128]) * 128 + c % 128
            valid = c < sp.n_cols[r] and tok < sp.row_ke[r] - sp.row_ks[r]
            if valid:
                assert lg[r, c] == dense[r, tok], f"row {r} col {c}"
            else:
                assert lg[r, c] == -np.inf, f"row {r} col {c} should be masked"


def pin_paged_sparse_equals_contiguous_sparse():
    """Candidate blocks read through a page table score exactly like the same candidate
    blocks of a contiguous row (same key bytes), for an identity and a permuted page pool,
    with and without a row -> request map, fp8 and MXFP4, ragged lengths and column
    counts (the last candidate block partly past the row)."""
    for kd, seed in (("fp8", 81), ("mxfp4", 82)):
        sp = synth.sparse_blocks(seed=seed, rows=4, ctx=2048, n_blocks=5, block=128, topk=50, kdtype=kd,
                                 ragged=True, poison_noncand=False)
        ref = O.logits_sparse(sp.q, "fp8", sp.w, sp.k, sp.k_scale, kd, sp.row_ks, sp.row_ke, sp.cand, sp.n_cols,
                              sp.block)
        for permute, row_req in ((False, False), (True, False), (True, True)):
            ps = synth.page_sparse(sp, page=64, seed=seed, permute=permute, row_req=row_req)
            got = O.logits_paged_sparse(ps.q, "fp8", ps.w, ps.k_pages, ps.k_scale_pages, kd, ps.block_table,
                                        ps.seq_lens, ps.cand, ps.n_cols, ps.block, row_req=ps.row_req)
            assert np.array_equal(got, ref), f"{kd} permute={permute} row_req={row_req}: paged-sparse != sparse"
        # 128-token pages hold whole candidate blocks (no split)
        ps = synth.page_sparse(sp, page=128, seed=seed, row_req=True)
        assert ps.block == 128
        got = O.logits_paged_sparse(ps.q, "fp8", ps.w, ps.k_pages, ps.k_scale_pages, kd, ps.block_table,
                                    ps.seq_lens, ps.cand, ps.n_cols, ps.block, row_req=ps.row_req)
        assert np.array_equal(got, ref), f"{kd}: 128-token pages"


def pin_paged_sparse_equals_paged_dense_masked():
    """Each scored candidate column equals the paged dense score of its token; every other
    column is -inf; and selecting over the candidate columns picks exactly what the paged
    dense route picks once non-candidate tokens are masked."""
    sp = synth.sparse_blocks(seed=83, rows=3, ctx=1024, n_blocks=4, block=128, topk=40, kdtype="fp8",
                             ragged=True, poison_noncand=False)
    ps = synth.page_sparse(sp, page=64, seed=83, row_req=True)
    lg = O.logits_paged_sparse(ps.q, "fp8", ps.w, ps.k_pages, ps.k_scale_pages, "fp8", ps.block_table,
                               ps.seq_lens, ps.cand, ps.n_cols, ps.block, row_req=ps.row_req)
    full = O.logits_paged(ps.q, "fp8", ps.w, ps.k_pages, ps.k_scale_pages, "fp8", ps.block_table, ps.seq_lens,
                          row_req=ps.row_req, ld=1024)
    mask = np.zeros_like(full, dtype=bool)
    assert ps.block == 64  # 128-token candidate blocks split over 64-token pages
    for r in range(ps.rows):
        for c in range(lg.shape[1]):
            tok = int(ps.cand[r, c // ps.block]) * ps.block + c % ps.block
            if c < ps.n_cols[r] and tok < ps.seq_lens[r]:
                assert lg[r, c] == full[r, tok], f"row {r} col {c}"
                mask[r, tok] = True
            else:
                assert lg[r, c] == -np.inf, f"row {r} col {c} should be masked"
    idx, val = O.select_case(ps, k=40)
    d_idx, d_val = O.topk(np.where(mask, full, -np.inf).astype(np.float32), 40)
    assert np.array_equal(idx, d_idx) and np.array_equal(val, d_val), "paged-sparse != paged dense-masked"


# ----------------------------------------------------------------------------- key-cache writer


def pin_fp8_encode_roundtrip_and_saturation():
    """Every finite e4m3fn value encodes to its own code; magnitudes just above 448 (as
    value * (448 / amax) can give) stay at 448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = torch_fp8(codes).astype(np.float32)
    got = O.encode_fp8(vals)
    assert np.array_equal(got, codes), "e4m3fn values do not encode to themselves"
    assert O.encode_fp8(np.float32(448.0) * np.float32(1 + 2 ** -23)) == 0x7E
    assert O.encode_fp8(-np.float32(460.0)) == 0xFE


def pin_fp8_encode_vs_torch():
    """Nearest-even e4m3fn encoding against torch's independent float8_e4m3fn cast, on
    random values and on every midpoint between neighbouring codes (the ties)."""
    rng = np.random.default_rng(81)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(1000) * 1e-2,
                        rng.standard_normal(500) * 2.0 ** -9]).astype(np.float32)
    pos = np.unique(np.abs(torch_fp8(np.arange(127, dtype=np.uint8))))
    mid = (pos[1:] + pos[:-1]) / 2
    mid = mid[mid.astype(np.float32).astype(np.float64) == mid].astype(np.float32)
    x = np.concatenate([x, mid, -mid])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_fp8(x), want), "e4m3fn encoding differs from torch"


def pin_e2m1_encode_ties():
    """e2m1 encoding from the OCP table: grid values to their codes, each midpoint of two
    neighbouring magnitudes to the neighbour with the even code, magnitudes above 6 to 6,
    negative values to the same magnitude code with the sign bit."""
    g = e2m1_golden()
    mags = sorted((v, c) for c, v in g.items() if c < 8)
    for v, c in mags:
        assert O.encode_e2m1(v) == c and O.encode_e2m1(-v) == (c | 8), f"grid value {v}"
    for (v0, c0), (v1, c1) in zip(mags, mags[1:]):
        even = c0 if c0 % 2 == 0 else c1
        assert O.encode_e2m1((v0 + v1) / 2) == even, f"tie between {v0} and {v1}"
        assert O.encode_e2m1(v0 + (v1 - v0) * 0.49) == c0 and O.encode_e2m1(v0 + (v1 - v0) * 0.51) == c1
    assert O.encode_e2m1(7.5) == 7 and O.encode_e2m1(-100.0) == 15


def _bf16_keys(rng, n):
    x = (rng.standard_normal((n, 128)) * rng.uniform(0.01, 10, (n, 1))).astype(np.float32)
    x[0] = 0.0                       # all zero
    x[1] = 0.0
    x[1, 5] = -3.0e-3                # one non-zero entry
    x[2, 17] = 3.0e4                 # one outlier
    x[3, :64] = np.float32(2.0 ** -130)  # subnormal magnitudes next to normal ones
    return synth.to_bf16_bits(x)


def _writer_case(kd, seed):
    rng = np.random.default_rng(seed)
    n, n_slots = 40, 64
    keys = _bf16_keys(rng, n)
    slots = rng.permutation(n_slots)[:n].astype(np.int64)
    slots[7] = -1                    # padding token: writes nothing
    slots[9] = n_slots + 3           # outside the cache: skipped and counted
    kb, sdt, sw = (128, np.float32, 1) if kd == "fp8" else (64, np.uint8, 4)
    cache = np.full((n_slots, kb), 0x5A, np.uint8)
    sc = np.full((n_slots, sw), 0x5A, np.uint8).view(sdt).reshape(n_slots, -1).copy() if kd != "fp8" \
        else np.full(n_slots, 1234.5, np.float32)
    bad = O.kcache_write(keys, slots, kd, cache, sc)
    return keys, slots, cache, sc, bad


def pin_kcache_fp8():
    """fp8 writer: scale = amax / 448 in float32, codes = torch's e4m3fn cast of
    value * (448 / amax), the largest element at +-448, padding and out-of-range slots
    untouched."""
    keys, slots, cache, sc, bad = _writer_case("fp8", 82)
    assert bad == 1
    x = torch_bf16(keys).astype(np.float32)
    for i, s in enumerate(slots):
        if s < 0 or s >= cache.shape[0]:
            continue
        amax = np.abs(x[i]).max()
        if amax == 0:
            assert sc[s] == 0 and np.all((cache[s] & 0x7F) == 0), f"zero key {i}"
            continue
        assert sc[s] == np.float32(amax) / np.float32(448.0), f"scale of key {i}"
        y = x[i] * (np.float32(448.0) / np.float32(amax))
        want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(cache[s], want), f"codes of key {i}"
        assert (cache[s][np.argmax(np.abs(x[i]))] & 0x7F) == 0x7E
    untouched = np.setdiff1d(np.arange(cache.shape[0]), slots[(slots >= 0) & (slots < cache.shape[0])])
    assert np.all(cache[untouched] == 0x5A) and np.all(sc[untouched] == np.float32(1234.5))


def pin_kcache_mxfp4():
    """MXFP4 writer: per group of 32 the UE8M0 byte is floor(log2 amax) - 2 + 127 (closed
    form from the exact value), every element decodes to within half a grid step of its
    value (saturating at 6 * 2^X), and the codes equal the input generator's separate
    OCP MX encoder."""
    keys, slots, cache, sc, bad = _writer_case("mxfp4", 83)
    assert bad == 1
    x = torch_bf16(keys)
    g = e2m1_golden()
    for i, s in enumerate(slots):
        if s < 0 or s >= cache.shape[0]:
            continue
        for grp in range(4):
            xs = x[i, 32 * grp: 32 * grp + 32]
            amax = float(np.abs(xs).max())
            X = (math.frexp(amax)[1] - 1 - 2) if amax > 0 else -127
            biased = min(max(X + 127, 0), 254)
            assert sc[s, grp] == biased, f"key {i} group {grp} scale"
            step = 2.0 ** (biased - 127)
            for j in range(32):
                b = cache[s, 16 * grp + j // 2]
                nib = (b & 0xF) if j % 2 == 0 else (b >> 4)
                v = g[int(nib)] * step
                t = min(abs(xs[j]), 6.0 * step)
                half = 0.25 * step if t < 2 * step else (0.5 * step if t < 4 * step else step)
                assert abs(abs(v) - t) <= half * (1 + 1e-12), f"key {i} element {32 * grp + j}"
        want_codes, want_sc = synth.to_mxfp4(torch_bf16(keys[i:i + 1]).astype(np.float32))
        assert np.array_equal(cache[s], want_codes[0]) and np.array_equal(sc[s], want_sc[0]), f"key {i}"
    untouched = np.setdiff1d(np.arange(cache.shape[0]), slots[(slots >= 0) & (slots < cache.shape[0])])
    assert np.all(cache[untouched] == 0x5A) and np.all(sc[untouched] == 0x5A)




# ----------------------------------------------------------------------------- sparse attention


def _bf16_bits(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _attn_case(seed, rows=3, H=16, n=150, pages=None):
    rng = np.random.default_rng(seed)
    q = _bf16_bits(rng.standard_normal((rows, H, 576)) * 0.08)
    P = pages if pages is not None else (n + 63) // 64
    kv = _bf16_bits(rng.standard_normal((rows * P, 64, 576)))
    bt = np.arange(rows * P, dtype=np.int32).reshape(rows, P)
    return q, kv, bt, np.full(rows, n, np.int32)


def pin_attn_single_entry():
    """One selected entry: softmax weight 1, the output is that entry's first 512 values."""
    q, kv, bt, sl = _attn_case(60)
    idx = np.array([[17, -1], [-1, 130], [5, 5000]], np.int32)
    out, lse = O.sparse_attn_paged(q, kv, bt, sl, idx, 0.1)
    vals = torch_bf16(kv).reshape(-1, 576)
    for r, s in enumerate([17, 130, 5]):
        assert np.array_equal(out[r], np.broadcast_to(vals[bt[r][s // 64] * 64 + s % 64][:512], (16, 512)).astype(np.float32))
    assert np.all(np.isfinite(lse))


def pin_attn_uniform_weights():
    """q = 0: every score is 0, the output is the mean of the selected values, lse = log n."""
    q, kv, bt, sl = _attn_case(61)
    q[:] = 0
    idx = np.array([[1, 2, 3, 64], [0, 149, -1, -1], [7, 8, 9, 10]], np.int32)
    out, lse = O.sparse_attn_paged(q, kv, bt, sl, idx, 0.3)
    vals = torch_bf16(kv).reshape(-1, 576).astype(np.float64)
    for r in range(3):
        sel = [s for s in idx[r] if s >= 0]
        mean = np.mean([vals[bt[r][s // 64] * 64 + s % 64][:512] for s in sel], axis=0)
        assert np.allclose(out[r], mean[None, :], rtol=1e-6, atol=1e-7)
        assert np.allclose(lse[r], np.log(len(sel)), rtol=1e-6)


def pin_attn_vs_sdpa():
    """Against torch's scaled-dot-product attention in float64 (an independent
    implementation): all positions selected, and a random subset through a boolean mask
    (so the result must use the selected positions, not the first k)."""
    q, kv, bt, sl = _attn_case(62, rows=2, H=16, n=128)
    scale = 0.06
    rng = np.random.default_rng(63)
    sub = np.sort(rng.choice(128, size=40, replace=False)).astype(np.int32)
    for r, sel in ((0, np.arange(128, dtype=np.int32)), (1, sub)):
        idx = np.full((2, 128), -1, np.int32)
        idx[r, :len(sel)] = rng.permutation(sel)
        out, lse = O.sparse_attn_paged(q, kv, bt, sl, idx, scale)
        vals = torch.from_numpy(torch_bf16(kv)[bt[r]].reshape(-1, 576).astype(np.float64))  # the row's 128 tokens
        qq = torch.from_numpy(torch_bf16(q[r]).astype(np.float64))[:, None, :]               # [H, 1, 576]
        mask = torch.zeros(128, dtype=torch.bool)
        mask[torch.from_numpy(sel.astype(np.int64))] = True
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, vals[None].expand(16, -1, -1), vals[None, :, :512].expand(16, -1, -1),
            attn_mask=mask[None, None, :].expand(16, 1, -1), scale=scale)[:, 0, :].numpy()
        assert np.allclose(out[r], ref, rtol=1e-5, atol=1e-6), f"row {r} differs from SDPA"
        z = (qq[:, 0, :] @ vals.T).numpy() * scale
        ref_lse = np.log(np.exp(z[:, sel]).sum(axis=1))
        assert np.allclose(lse[r], ref_lse, rtol=1e-6)


def pin_attn_index_order_and_padding():
    """The selection is a set: permuting it, or adding -1 / out-of-range entries, changes
    nothing."""
    q, kv, bt, sl = _attn_case(64)
    rng = np.random.default_rng(65)
    base = np.stack([np.sort(rng.choice(150, 30, replace=False)) for _ in range(3)]).astype(np.int32)
    a, la = O.sparse_attn_paged(q, kv, bt, sl, base, 0.09)
    shuf = np.stack([rng.permutation(b) for b in base])
    padded = np.concatenate([shuf, np.full((3, 5), -1, np.int32), np.full((3, 2), 150, np.int32)], axis=1)
    b, lb = O.sparse_attn_paged(q, kv, bt, sl, padded, 0.09)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7) and np.allclose(la, lb, rtol=1e-6)


def pin_attn_paged_equals_contiguous():
    """A permuted page table over permuted pages gives the contiguous result."""
    q, kv, bt, sl = _attn_case(66)
    rng = np.random.default_rng(67)
    idx = np.stack([rng.choice(150, 40, replace=False) for _ in range(3)]).astype(np.int32)
    a, la = O.sparse_attn_paged(q, kv, bt, sl, idx, 0.05)
    perm = rng.permutation(kv.shape[0])
    kv2 = np.empty_like(kv)
    kv2[perm] = kv
    bt2 = perm[bt].astype(np.int32)
    b, lb = O.sparse_attn_paged(q, kv2, bt2, sl, idx, 0.05)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
