"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that at least
one pin fails for each: the pins are strong enough to notice a dropped term, a wrong
sign, bias or index, or a transposed operand."""
import subprocess
from pathlib import Path

import pytest

import oracle
import oracle_pins as pins

SRC = Path(oracle.__file__).resolve().parent / "ref.c"

MUTANTS = {
    "relu_dropped": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "weight_index": ("acc += (double)w[j] * relu;", "acc += (double)w[0] * relu;"),
    "weight_sign": ("acc += (double)w[j] * relu;", "acc -= (double)w[j] * relu;"),
    "head_index": ("dot += qd[(int64_t)j * dim + i] * kd[i];", "dot += qd[i] * kd[i];"),
    "q_transposed": ("dot += qd[(int64_t)j * dim + i] * kd[i];",
                     "dot += qd[(int64_t)(i % heads) * dim + (j + i) % dim] * kd[i];"),
    "fp8_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_subnormal": ("mag = ldexp((double)m / 8.0, 1 - 7);", "mag = ldexp((double)m / 8.0, -7);"),
    "fp8_mantissa": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 16.0, e - 7);"),
    "fp8_nan": ("if (e == 15 && m == 7)\n        return NAN;", "if (e == 15 && m == 7 && sign)\n        return NAN;"),
    "nibble_order": ("(i % 2 == 0) ? (byte & 0xF) : (byte >> 4)", "(i % 2 == 1) ? (byte & 0xF) : (byte >> 4)"),
    "e2m1_bias": ("mag = ldexp(1.0 + (double)m / 2.0, e - 1);", "mag = ldexp(1.0 + (double)m / 2.0, e - 2);"),
    "ue8m0_bias": ("return ldexp(1.0, (int)e - 127);", "return ldexp(1.0, (int)e - 128);"),
    "scale_group": ("ref_decode_ue8m0(((const uint8_t*)sc)[i / 32])", "ref_decode_ue8m0(((const uint8_t*)sc)[(i / 32) ^ 1])"),
    "scale_ignored": ("out[i] = ref_decode_fp8_e4m3fn(k[i]) * (double)*(const float*)sc;",
                      "out[i] = ref_decode_fp8_e4m3fn(k[i]);"),
    "bf16_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "double_rounding": ("return (float)acc;", "return (float)(double)(float)(acc * (1.0 + 1e-7));"),
    "dense_range_start": ("int64_t s = row_ks[r] + c;", "int64_t s = c;"),
    "dense_length": ("int64_t len = (int64_t)row_ke[r] - row_ks[r];\n        for (int64_t c = 0; c < ld; c++) {\n            if (c >= len) {\n                logits[r * ld + c] = -INFINITY;",
                     "int64_t len = (int64_t)row_ke[r] - row_ks[r] + 1;\n        for (int64_t c = 0; c < ld; c++) {\n            if (c >= len) {\n                logits[r * ld + c] = -INFINITY;"),
    "paged_slot": ("int64_t slot = page * page_size + s % page_size;", "int64_t slot = page * page_size + (s + 1) % page_size;"),
    "paged_req": ("int64_t req = row_req ? row_req[r] : r;", "int64_t req = r;"),
    "sparse_token": ("(int64_t)cand[r * cand_ld + b] * block + c % block", "(int64_t)cand[r * cand_ld + b] * block + (c + 1) % block"),
    "sparse_end": ("if (c >= n_cols[r] || b >= cand_ld", "if (c > n_cols[r] || b >= cand_ld"),
    "tie_break": ("return (a->idx > b->idx) - (a->idx < b->idx);", "return (a->idx < b->idx) - (a->idx > b->idx);"),
    "ascending": ("if (a->v > b->v)\n        return -1;\n    if (a->v < b->v)\n        return 1;",
                  "if (a->v < b->v)\n        return -1;\n    if (a->v > b->v)\n        return 1;"),
    "neg_inf_selected": ("if (isnan(v) || v == -INFINITY)", "if (isnan(v))"),
    "topk_len": ("int64_t n = lens ? lens[r] : ncols;", "int64_t n = ncols;"),
    "fp8_enc_ties_odd": ("if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));",
                         "if (d < best_d || (d == best_d && (c & 1) == 1 && (best & 1) == 0)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(best | (signbit(y) ? 0x80 : 0));"),
    "fp8_enc_sign": ("return (uint8_t)(best | (signbit(y) ? 0x80 : 0));", "return (uint8_t)best;"),
    "e2m1_enc_ties_odd": ("if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(best | (signbit(v) ? 8 : 0));",
                          "if (d < best_d || (d == best_d && (c & 1) == 1 && (best & 1) == 0)) {\n            best = c;\n            best_d = d;\n        }\n    }\n    return (uint8_t)(best | (signbit(v) ? 8 : 0));"),
    "writer_scale_inverted": ("*(float*)scale = amax / 448.0f;", "*(float*)scale = 448.0f / amax;"),
    "writer_fp8_max": ("float inv = 448.0f / amax;", "float inv = 240.0f / amax;"),
    "writer_mx_exponent": ("X = (e - 1) - 2;", "X = (e - 1) - 1;"),
    "writer_mx_nibbles": ("codes[16 * g + i / 2] = (uint8_t)(lo | (hi << 4));", "codes[16 * g + i / 2] = (uint8_t)(hi | (lo << 4));"),
    "cand_first_not_max": ("if (!have || v > best)", "if (!have)"),
    "cand_min_not_max": ("if (!have || v > best)", "if (!have || v < best)"),
    "cand_partial_block_dropped": ("const int64_t nblk = (n + block - 1) / block;", "const int64_t nblk = n / block;"),
    "cand_selection_order": ("if (chosen[b])\n                cand[r * cand_ld + o++] = (int32_t)b;",
                             "if (b < take)\n                cand[r * cand_ld + o++] = buf[b].idx;"),
    "cand_absent_counted": ("if (!(v > -INFINITY)) /* -inf or NaN */", "if (isnan(v))"),
    "cand_lens_ignored": ("int64_t n = lens ? lens[r] : ncols;\n        if (n < 0)", "int64_t n = ncols;\n        if (n < 0)"),
    "writer_padding_slot": ("if (s < 0)\n            continue;", "if (s < 0)\n            s = 0;"),
    "paged_sparse_token": ("(int64_t)cand[r * cand_ld + b] * block + c % block : -1;\n            if (c >= n_cols[r] || b >= cand_ld || tok < 0 || tok >= seq_lens[r])",
                           "(int64_t)cand[r * cand_ld + b] * block + (c + 1) % block : -1;\n            if (c >= n_cols[r] || b >= cand_ld || tok < 0 || tok >= seq_lens[r])"),
    "paged_sparse_len": ("tok < 0 || tok >= seq_lens[r])", "tok < 0 || tok > seq_lens[r])"),
    "paged_sparse_page_by_column": ("int64_t page = block_table[req * bt_ld + tok / page_size];",
                                    "int64_t page = block_table[req * bt_ld + c / page_size];"),
    "paged_sparse_slot": ("int64_t slot = page * page_size + tok % page_size;",
                          "int64_t slot = page * page_size + (tok + 1) % page_size;"),
    "paged_sparse_req": ("int64_t req = row_req ? row_req[r] : r;\n        for (int64_t c = 0; c < ld; c++) {\n            int64_t b = c / block;",
                         "int64_t req = r;\n        for (int64_t c = 0; c < ld; c++) {\n            int64_t b = c / block;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, mutant_dir, oracle_lib):
    old, new = MUTANTS[name]
    src = SRC.read_text()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = mutant_dir / f"{name}.c"
    mut.write_text(src.replace(old, new, 1))
    so = mutant_dir / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", str(mut), "-o", str(so), "-lm"], check=True)
    failed = []
    with oracle.variant(so):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except AssertionError:
                failed.append(pin.__name__)
                break
    assert failed, f"no pin caught the planted mistake {name}"


# The sparse-attention oracle is numpy code: its mutants are copies of the function with
# one planted mistake each, swapped in for the pins.
ATTN_MUTANTS = {
    "attn_scale_dropped": ("z = scale * (q[r] @ c.T)", "z = (q[r] @ c.T)"),
    "attn_value_slice": ("out[r] = (e / den) @ c[:, :512]", "out[r] = (e / den) @ c[:, 64:]"),
    "attn_first_k": ("pos = [int(s) for s in idx[r] if 0 <= s < seq_lens[r]]",
                     "pos = list(range(sum(1 for s in idx[r] if 0 <= s < seq_lens[r])))"),
    "attn_padding_kept": ("pos = [int(s) for s in idx[r] if 0 <= s < seq_lens[r]]",
                          "pos = [int(s) for s in idx[r] if s < seq_lens[r]]"),
    "attn_page_slot": ("bt[req][s // page_size], s % page_size]", "bt[req][s // page_size], (s + 1) % page_size]"),
    "attn_not_normalised": ("out[r] = (e / den) @ c[:, :512]", "out[r] = e @ c[:, :512]"),
    "attn_lse_without_max": ("lse[r] = (m + np.log(den))[:, 0]", "lse[r] = np.log(den)[:, 0]"),
}


@pytest.mark.parametrize("name", sorted(ATTN_MUTANTS))
def test_planted_attention_mistake_is_caught(name, monkeypatch, oracle_lib):
    import inspect
    import textwrap
    old, new = ATTN_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.sparse_attn_paged))
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new, 1), f"<{name}>", "exec"), ns)
    monkeypatch.setattr(oracle, "sparse_attn_paged", ns["sparse_attn_paged"])
    failed = []
    for pin in [p for p in pins.ALL_PINS if p.__name__.startswith("pin_attn")]:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches {name}"
