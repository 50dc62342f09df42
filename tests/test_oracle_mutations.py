"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.  The real oracle passes all pins
(test_oracle.py); each mutant here must fail at least one.

Not listed: swapping the MXFP4 nibble order (or any other permutation of the
elements inside one 32-element block) in the shared decoder.  Applied to Q and
K alike it permutes the terms of every dot product and leaves every score
unchanged, so no output can reveal it; the nibble convention is an ABI choice,
probed one-sidedly on the GPU by the layout pins."""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (id, text in oracle.c, replacement, which occurrence (0-based) to replace)
MUTANTS = [
    ("relu_dropped", "double relu = dot[h] > 0.0 ? dot[h] : 0.0;", "double relu = dot[h];", 0),
    ("relu_wrong_side", "double relu = dot[h] > 0.0 ? dot[h] : 0.0;", "double relu = dot[h] < 0.0 ? dot[h] : 0.0;", 0),
    ("weight_dropped", "acc += wd[h] * relu;", "acc += relu;", 0),
    ("weight_abs", "acc += wd[h] * relu;", "acc += fabs(wd[h]) * relu;", 0),
    ("sm_scale_dropped", "out[j] = sm_scale * acc;", "out[j] = acc;", 0),
    ("k_scale_byte_reversed", "word >> (8 * (d / 32))", "word >> (8 * (3 - d / 32))", 0),
    ("q_scale_byte_reversed", "word >> (8 * (d / 32))", "word >> (8 * (3 - d / 32))", 1),
    ("e4m3_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", 0),
    ("e4m3_subnormal", "ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)", 0),
    ("e2m1_subnormal", "v = 0.5 * (double)m;", "v = (double)m;", 0),
    ("e2m1_bias", "ldexp(1.0 + 0.5 * (double)m, e - 1)", "ldexp(1.0 + 0.5 * (double)m, e - 2)", 0),
    ("fp8_row_scale_dropped", "if (fmt == OR_FP8) v *= (double)((const float*)k_scale_b)[j];", "", 0),
    ("window_off_by_one", "+ (int64_t)i + 1;", "+ (int64_t)i;", 0),
    ("window_no_end_clamp", "if (e < s) e = s;", "", 0),
    ("window_start_ignored", "if (j < s || j >= e) {", "if (j >= e) {", 0),
    ("q_transposed", "Qt[(size_t)d * H + h] = v;", "Qt[(size_t)h * D + d] = v;", 0),
    ("k_batch_ignored", "const double* kj = Kd + ((size_t)b * S_k + j) * D;", "const double* kj = Kd + (size_t)j * D;", 0),
    ("w_bf16_read_as_f32", "(w_fmt == OR_W_F32)", "(1)", 0),
    ("dot_not_reset", "for (int h = 0; h < H; ++h) dot[h] = 0.0;", "", 0),
    ("bound_without_k_norm", "fabs(sm_scale) * kn[(size_t)b * S_k + j] * bs", "fabs(sm_scale) * bs", 0),
    ("paged_row_in_page", "row = page * page_size + j % page_size;", "row = page * page_size + j / page_size;", 0),
    ("paged_request_ignored", "block_table[(int64_t)b * max_pages + j / page_size]", "block_table[j / page_size]", 0),
    ("paged_window_off_by_one", "int64_t e = n - S_q + i + 1;", "int64_t e = n - S_q + i;", 0),
    ("paged_context_not_cut", "if (j < n) {", "if (j < S_k) {", 0),
    ("thd_visible_off_by_one", "e = s + (t + 1) / ratio", "e = s + t / ratio", 0),
    ("thd_visible_ceil", "e = s + (t + 1) / ratio", "e = s + (t + ratio) / ratio", 0),
    ("thd_no_segment_clamp", "if (e > lim) e = lim;", "", 0),
    ("thd_start_global", "int64_t s = cu_k[seg],", "int64_t s = cu_k[0],", 0),
    ("topk_ascending", "if (a->v > b->v) return -1;", "if (a->v < b->v) return -1;", 0),
    ("topk_ties_to_larger_column", "return (a->j > b->j) - (a->j < b->j);", "return (a->j < b->j) - (a->j > b->j);", 0),
    ("topk_nan_first", "if (an != bn) return an ? 1 : -1;", "if (an != bn) return an ? -1 : 1;", 0),
    ("topk_window_start_ignored", "for (int32_t j = s; j < e; ++j) {", "for (int32_t j = 0; j < e; ++j) {", 0),
    ("topk_padding_score_zero", "val[r * k + t] = -INFINITY;", "val[r * k + t] = 0.0f;", 0),
    ("topk_by_column_sorts_all", "qsort(c, (size_t)(n < k ? n : k), sizeof(or_cand), or_by_column);",
     "qsort(c, (size_t)n, sizeof(or_cand), or_by_column);", 0),
    ("topk_by_column_ignored", "if (by_column) qsort(", "if (0) qsort(", 0),
]


def _mutate(src: str, old: str, new: str, nth: int) -> str:
    pos = -1
    for _ in range(nth + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r} (occurrence {nth})"
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("mid,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, old, new, nth):
    src = open(oracle.SRC).read()
    mutated = _mutate(src, old, new, nth)
    assert mutated != src
    cpath = os.path.join(tmp_path, f"{mid}.c")
    with open(cpath, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(cpath, os.path.join(tmp_path, f"lib{mid}.so"))
    orc = oracle.Oracle(lib)
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:
            return  # caught
    pytest.fail(f"no pin caught mutant {mid}")
