"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Every mutant is a textual edit of ``oracle/losa_oracle.c`` compiled into a
temporary library on the CPU; the pins of ``oracle_pins`` run against it and
at least one must fail.  This shows that the pins would notice a dropped term,
a wrong sign, index or operand anywhere in the oracle.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins as P
from oracle import build as obuild

# (name, original text, replacement, which occurrence (0-based) or None for all)
MUTANTS = [
    ("locality_sign", "float delta = a[i] - b[i];", "float delta = a[i] + b[i];", None),
    ("locality_dropped_sum", "acc = acc + sq;", "acc = sq;", None),
    ("locality_no_mean", "score[((int64_t)s * H + h) * B + t] = acc / (float)d;",
     "score[((int64_t)s * H + h) * B + t] = acc;", None),
    ("active_order", "sc[t] > sc[best]", "sc[t] < sc[best]", None),
    ("active_tie_break", "sc[t] > sc[best]", "sc[t] >= sc[best]", None),
    ("meta_max", "if (v > hi) hi = v;", "if (v < hi) hi = v;", None),
    ("meta_partial_page", "if (t1 > prefix_len[s]) t1 = prefix_len[s];", "", None),
    ("bound_min_max_swapped", "q[i] >= 0.0f ? mx[i] : mn[i]", "q[i] >= 0.0f ? mn[i] : mx[i]", None),
    ("bound_dropped_sum", "acc = acc + prod;", "acc = prod;", None),
    ("bound_sign_rule", "q[i] >= 0.0f ? mx[i] : mn[i]", "q[i] < 0.0f ? mx[i] : mn[i]", None),
    ("topk_tie_break", "U[p] > U[best]", "U[p] >= U[best]", None),
    ("topk_order", "U[p] > U[best]", "U[p] < U[best]", None),
    ("row_to_head", "const int h = g * G + r / A, a = r % A;", "const int h = g + r / A, a = r % A;",
     None),
    ("score_scale", "s_buf[j] = scale * dot;", "s_buf[j] = dot;", None),
    ("lse_max", "*lse = m + log(sum);", "*lse = log(sum);", None),
    ("merge_weights_swapped", "o[i] = wp * op[i] + ws * os[i];", "o[i] = ws * op[i] + wp * os[i];",
     None),
    ("suffix_keys_are_values", "keys[u] = k_blk + ", "keys[u] = v_blk + ", None),
    ("prefix_mask_dropped", "if (t >= prefix_len[s]) break;", "", None),
    ("bf16_rounding_bits", "int q = e - 8;", "int q = e - 9;", None),
    ("suffix_kv_head", "const int g = h / G;\n            for (int u = 0;",
     "const int g = h % Hk;\n            for (int u = 0;", None),
    ("dense_kv_head", "prefix_attend(sh, s, h / G,", "prefix_attend(sh, s, h % Hk,", None),
    ("stable_rows_zeroed", "    suffix_and_merge(sh, q_t, k_blk, v_blk, op_use, lp_use, out);\n",
     "    for (int s2 = 0; s2 < sh->n_seq * H * B; ++s2) { int keep = 0;\n"
     "        for (int a2 = 0; a2 < A; ++a2) if (active[(s2 / B) * A + a2] == s2 % B) keep = 1;\n"
     "        if (!keep) { lp_use[s2] = -INFINITY; } }\n"
     "    suffix_and_merge(sh, q_t, k_blk, v_blk, op_use, lp_use, out);\n",
     None),
    ("shared_dropped_head", "for (int h = 0; h < H; ++h) acc = acc + score[",
     "for (int h = 1; h < H; ++h) acc = acc + score[", None),
    ("shared_max_not_sum", "acc = acc + score[((int64_t)s * H + h) * B + t];",
     "acc = fmaxf(acc, score[((int64_t)s * H + h) * B + t]);", None),
    ("shared_set_ignored", "if (sh->flags & ORACLE_SHARED_ACTIVE) {", "if (0) {", None),
    ("row_mask_ignored", "if (sh->flags & ORACLE_ROW_MASK) {", "if (0) {", None),
    ("no_writeback_ignored", "if (sh->flags & ORACLE_NO_WRITEBACK) {", "if (0) {", None),
    ("locality_chain_reversed", "for (int i = 0; i < d; ++i) {\n                    float delta",
     "for (int i = d - 1; i >= 0; --i) {\n                    float delta", None),
    ("locality_chain_in_double",
     "float acc = 0.0f;\n                for (int i = 0; i < d; ++i) {\n                    float delta",
     "double acc = 0.0;\n                for (int i = 0; i < d; ++i) {\n                    float delta",
     None),
    ("bound_chain_reversed", "for (int i = 0; i < d; ++i) {\n        float sel",
     "for (int i = d - 1; i >= 0; --i) {\n        float sel", None),
    ("bound_chain_in_double", "    float acc = 0.0f;\n    for (int i = 0; i < d; ++i) {\n        float sel",
     "    double acc = 0.0;\n    for (int i = 0; i < d; ++i) {\n        float sel", None),
]


def _mutate(src: str, old: str, new: str, which):
    n = src.count(old)
    assert n >= 1, f"mutation anchor not found: {old!r}"
    if which is None:
        return src.replace(old, new)
    parts = src.split(old)
    return old.join(parts[: which + 1]) + new + old.join(parts[which + 1:])


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,which", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, tmp_path, name, old, new, which):
    src = _mutate(source, old, new, which)
    c_path = tmp_path / f"mut_{name}.c"
    c_path.write_text(src)
    so_path = str(tmp_path / f"libmut_{name}.so")
    obuild.build(str(c_path), so_path)
    lib = oracle.load(so_path)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
            break
    assert failed, f"mutant {name} passed every pin"
