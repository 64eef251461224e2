"""Plant a plausible mistake in a copy of the oracle (on the CPU) and check that
at least one pin catches it.  This is how the pins are shown to cover the
oracle: a dropped term, a wrong sign, index or operand must not pass."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = [
    ("dropped_scale", "s[p] = scale * dot + mask[(size_t)j * nk + p];",
     "s[p] = dot + mask[(size_t)j * nk + p];"),
    ("gqa_head_map", "if (h / G != g) continue;", "if (h % num_kv_heads != g) continue;"),
    ("prefix_mask_off_by_one", "int vis = (p < L) ||", "int vis = (p + 1 < L) ||"),
    ("mask_excludes_self", "    int a = j;\n", "    int a = parent_of(tree_parent, o, j);\n"),
    ("missing_normaliser", "const double w = s[p] / z;", "const double w = s[p];"),
    ("slot_layout_transposed",
     "(((long long)page * num_kv_heads + g) * page_size + (p % page_size))",
     "(((long long)page * page_size + (p % page_size)) * num_kv_heads + g)"),
    ("bf16_widening", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    ("argmax_last_tie", "if (x[v] > x[best]) best = v;", "if (x[v] >= x[best]) best = v;"),
    ("chain_wrong_index", "draft[o + n + 1] == target[o + n]", "draft[o + n + 1] == target[o + n + 1]"),
    ("tree_tie_break", "if (acc[j] && depth[j] > depth[best]) best = j;",
     "if (acc[j] && depth[j] >= depth[best]) best = j;"),
    ("tree_ignores_ancestors", "acc[j] = acc[p] && draft[o + j] == target[o + p];",
     "acc[j] = draft[o + j] == target[o + p];"),
    ("out_tokens_index", "out_tokens[o + k] = target[o + path[k]];", "out_tokens[o + k] = target[o + k];"),
    ("compact_source", "const int src = L + accepted_path[cu_q[i] + k];", "const int src = L + k;"),
    ("compact_new_len", "new_context_lens[i] = context_lens[i] + accept_len[i];",
     "new_context_lens[i] = context_lens[i] + accept_len[i] - 1;"),
    ("decode_range", "const int nk = pos + 1;", "const int nk = pos;"),
    ("softmax_sign", "s[p] = exp(s[p] - m); /* masked: exp(-inf) = 0 */",
     "s[p] = exp(m - s[p]); /* masked: exp(-inf) = 0 */"),
    ("chunk_alive_own_edge_only", "for (int a = j; a > 0; a = parent_of(tree_parent, o, a)) {",
     "for (int a = j; a == j && a > 0; a = parent_of(tree_parent, o, a)) {"),
    ("chunk_skips_first_unverified", "for (int j = e; j < qn && !go_on; ++j)",
     "for (int j = e + 1; j < qn && !go_on; ++j)"),
    ("chunk_next_len_unclamped", "next_len[i] = qn - e < chunk_size ? qn - e : chunk_size;",
     "next_len[i] = chunk_size;"),
    ("chunk_tie_break", "if (acc[j] && depth[j] > depth[best]) { best = j; }",
     "if (acc[j] && depth[j] >= depth[best]) { best = j; }"),
    ("chunk_next_begin_overlaps", "next_begin[i] = e;\n            next_len[i] = qn - e",
     "next_begin[i] = e - 1;\n            next_len[i] = qn - e"),
]


def test_mutations_apply_once():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    mutated = src.replace(old, new)
    assert mutated != src
    c_path = tmp_path / f"oracle_{name}.c"
    so_path = tmp_path / f"liboracle_{name}.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(c_path), "-o",
                           str(so_path), "-lm"])
    caught = None
    with oracle.use_library(str(so_path)):
        for check in pins.ALL_CHECKS:
            try:
                check()
            except (AssertionError, oracle.OracleError, ValueError, FloatingPointError) as e:
                caught = (check.__name__, e)
                break
    assert caught is not None, f"no pin caught mutant {name}"
