"""Plant plausible mistakes into copies of the oracle's C source (on the CPU)
and require each one to break at least one pin: evidence that the pins would
catch a dropped term, a wrong sign or index, or a transposed operand."""
import os
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to find (must occur exactly once), replacement)
MUTANTS = [
    ("scale_1_over_d", "1.0 / sqrt((double)d)", "1.0 / (double)d"),
    ("scale_missing", "s[e] = acc * scale;", "s[e] = acc;"),
    ("q_dot_q", "load(Q, dtype, qbase + c) * load(K, dtype, kbase + c)", "load(Q, dtype, qbase + c) * load(Q, dtype, kbase + c)"),
    ("v_of_query_row", "int64_t vbase = (bh * m->L + keys[e]) * d;", "int64_t vbase = (bh * m->L + q) * d;"),
    ("empty_row_nan", "if (n == 0) continue;", ""),
    ("exp_sign", "double w = exp(s[e] - mx);", "double w = exp(mx - s[e]);"),
    ("den_count", "for (int c = 0; c < d; ++c) o[c] /= den;", "for (int c = 0; c < d; ++c) o[c] /= (double)n;"),
    ("tm_inverse_swapped", "int64_t jq = logical_pos(m, h, q), jk = logical_pos(m, h, k);",
     "int64_t jq = token_of(m, h, q), jk = token_of(m, h, k);"),
    ("tm_formula", "return p * m->T + t;", "return t * m->T + p;"),
    ("block_col_by_bq", "return m->block_u8[(bh * nqb + jq / m->bq) * nkb + jk / m->bk] != 0;",
     "return m->block_u8[(bh * nqb + jq / m->bq) * nkb + jk / m->bq] != 0;"),
    ("block_transposed", "return m->block_u8[(bh * nqb + jq / m->bq) * nkb + jk / m->bk] != 0;",
     "return m->block_u8[(bh * nqb + jk / m->bq) * nkb + jq / m->bk] != 0;"),
    ("bits_word", "return (int)((m->block_bits[(bh * nqb + jq / m->bq) * words + kb / 64] >> (kb % 64)) & 1u);",
     "return (int)((m->block_bits[(bh * nqb + jq / m->bq) * words + kb / 64] >> (kb % 32)) & 1u);"),
    ("spatial_anchor_of_query", "return tk == tq || tk == m->anchor;", "return tk == tq || tq == m->anchor;"),
    ("spatial_no_anchor", "return tk == tq || tk == m->anchor;", "return tk == tq;"),
    ("temporal_strict", "return llabs(yk - yq) <= m->radius && llabs(xk - xq) <= m->radius;",
     "return llabs(yk - yq) < m->radius && llabs(xk - xq) <= m->radius;"),
    ("temporal_x_uses_y", "int64_t yk = (k % HW) / m->Wg, xk = (k % HW) % m->Wg;",
     "int64_t yk = (k % HW) / m->Wg, xk = (k % HW) / m->Wg;"),
    ("slice_no_layout", "int64_t list = ((int64_t)b * m->H + h) * nqb + logical_pos(m, h, q) / m->bq;",
     "int64_t list = ((int64_t)b * m->H + h) * nqb + q / m->bq;"),
    ("slice_key_not_mapped", "keys[n++] = (int32_t)token_of(m, h, m->col_idx[e]);", "keys[n++] = (int32_t)m->col_idx[e];"),
    ("bf16_low_half", "uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;",
     "uint32_t bits = (uint32_t)((const uint16_t *)p)[idx];"),
    ("count_no_crop", "if (on) total += rq * ((j + 1) * m->bk < m->L ? m->bk : m->L - j * m->bk);",
     "if (on) total += rq * m->bk;"),
    ("union_last_logical_block", "for (int64_t i = j0 / m->bq; i <= (j1 - 1) / m->bq; ++i)",
     "for (int64_t i = j0 / m->bq; i < (j1 - 1) / m->bq; ++i)"),
    ("union_no_crop", "if (any[kb]) total += (kb + 1) * m->bk < m->L ? m->bk : m->L - kb * m->bk;",
     "if (any[kb]) total += m->bk;"),
    ("union_rows_not_mapped", "int64_t n = om_row_keys(m, b, h, token_of(m, h, j), keys);",
     "int64_t n = om_row_keys(m, b, h, j, keys);"),
    ("union_block_end", "int64_t hi = (blk + 1) * M < m->L ? (blk + 1) * M : m->L;",
     "int64_t hi = (blk + 1) * M - 1 < m->L ? (blk + 1) * M - 1 : m->L;"),
]


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl, workdir):
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for {name} not unique/present"
    msrc = os.path.join(workdir, f"{name}.c")
    with open(msrc, "w") as f:
        f.write(src.replace(find, repl))
    mlib = oracle.build(src=msrc, out=os.path.join(workdir, f"lib_{name}.so"))
    broken = []
    for pin in pins.ALL_PINS:
        try:
            if pin(mlib):
                broken.append(pin.__name__)
        except Exception as e:  # a crash or shape error also counts as caught
            broken.append(f"{pin.__name__}:{type(e).__name__}")
        if broken:
            break
    assert broken, f"mutant {name} passed every pin"
