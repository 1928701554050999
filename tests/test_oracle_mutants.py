"""Plausible mistakes planted in copies of the oracle (on the CPU) must each be
caught by at least one pin.  This shows the pins constrain every part of the
oracle: a dropped term, a wrong index, a transposed layout or a wrong tie rule
anywhere fails a pin.  The real oracle source is never modified."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sv_oracle.c")

# (name, original text, replacement, occurrence index to replace)
MUTANTS = [
    ("mask_without_self", "int j = i;\n                while (j != -1) {",
     "int j = par[i];\n                while (j != -1) {", 0),
    ("mask_depth_off_by_one", "steps -= 1;", "steps -= 0;", 0),
    ("tree_second_root_allowed", "par[i] < 0 || par[i] >= i", "par[i] < -1 || par[i] >= i", 0),
    ("gqa_modulo_map", "const int kvh = h / G;", "const int kvh = h % Hkv;", 0),
    ("scale_dropped_on_prefix", "s[n] = scale * dot;", "s[n] = dot;", 0),
    ("prefix_off_by_one", "for (int64_t p = 0; p < P; ++p)",
     "for (int64_t p = 0; p + 1 < P; ++p)", 0),
    ("tree_mask_ignored", "if (!((mrow[j / 64] >> (j % 64)) & 1)) continue;", "", 0),
    ("output_layout_head_major", "dst = out + (((int64_t)b * T + i) * Hq + h) * D;",
     "dst = out + (((int64_t)b * Hq + h) * T + i) * D;", 0),
    ("softmax_weight_dropped", "num[d] += w * elem(vsrc[k], dtype, voff[k] + d);",
     "num[d] += elem(vsrc[k], dtype, voff[k] + d);", 0),
    ("values_read_from_keys", "vsrc[n] = v_cache;", "vsrc[n] = k_cache;", 0),
    ("tree_rows_from_head0", "int64_t off = (((int64_t)b * Hkv + kvh) * T + j) * D;",
     "int64_t off = (((int64_t)b * Hkv) * T + j) * D;", 0),
    ("argmax_ties_to_last", "best < 0 || x[v] > bv", "best < 0 || x[v] >= bv", 0),
    ("argmax_nan_not_skipped", "if (isnan(x[v])) continue;", "", 0),
    ("argmax_all_nan_minus_one", "return best < 0 ? 0 : (int32_t)best;",
     "return (int32_t)best;", 0),
    ("accept_compares_own_argmax", "drf[i] == a[par[i]]", "drf[i] == a[i]", 0),
    ("accept_ignores_parent_match", "match[par[i]] && drf[i] == a[par[i]]",
     "drf[i] == a[par[i]]", 0),
    ("accept_emits_drafts", "toks[j] = a[path[j]];", "toks[j] = drf[path[j]];", 0),
    ("accept_ties_to_largest", "match[i] && dep[i] > dep[best]",
     "match[i] && dep[i] >= dep[best]", 0),
    ("accept_ignores_tree_err", "(tree_err && tree_err[b] != 0) ||", "0 ||", 0),
    ("sampled_no_renormalise", "R -= px;", "", 0),
    ("sampled_rejected_token_drawn", "if (excl[y] || p[y] <= 0.0) continue;",
     "if (p[y] <= 0.0) continue;", 0),
    ("sampled_repeated_token_retried", "const double px = (in_vocab && !excl[x]) ? p[x] : 0.0;",
     "const double px = in_vocab ? p[x] : 0.0;", 0),
    ("sampled_compare_le", "* R < px) {", "* R <= px) {", 0),
    ("sampled_root_row_only", "const float *row = logits + ((int64_t)b * T + v) * V;",
     "const float *row = logits + ((int64_t)b * T) * V;", 0),
    ("sampled_temperature_ignored", "exp((l - m) / tau)", "exp(l - m)", 0),
    ("sampled_children_reversed", "for (int c = v + 1; c < T && next < 0; ++c) {",
     "for (int c = T - 1; c > v && next < 0; --c) {", 0),
    ("sampled_emits_parent_token", "toks[L - 1] = drf[next];", "toks[L - 1] = drf[v];", 0),
    ("sampled_uniform_of_parent", "u_accept[(int64_t)b * T + c]", "u_accept[(int64_t)b * T + v]", 0),
    ("sampled_draw_not_scaled", "const double target = (double)u_sample[(int64_t)b * T + v] * R;",
     "const double target = (double)u_sample[(int64_t)b * T + v];", 0),
    ("sampled_nan_counts", "if (isnan(x)) return -INFINITY;", "", 0),
    ("sampled_ignores_tree_err", "(tree_err && tree_err[b] != 0) ||", "0 ||", 1),
    ("rope_gptj_pairs", "const double x1 = elem(x, dtype, row + j), x2 = elem(x, dtype, row + j + half);",
     "const double x1 = elem(x, dtype, row + (2 * j) % D), x2 = elem(x, dtype, row + (2 * j + 1) % D);", 0),
    ("rope_frequency_exponent", "pow(theta, -2.0 * (double)j / (double)D)", "pow(theta, -(double)j / (double)D)", 0),
    ("rope_sign", "x1 * c - x2 * sn", "x1 * c + x2 * sn", 0),
    ("rope_position_is_index", "(double)prefix_len[b] + (double)depth[(int64_t)b * T + i]",
     "(double)prefix_len[b] + (double)i", 0),
    ("rope_prefix_ignored", "(double)prefix_len[b] + (double)depth[(int64_t)b * T + i]",
     "(double)depth[(int64_t)b * T + i]", 0),
    ("rope_keys_not_rotated", "    rope_rows(k_tree, dtype, Hkv, prefix_len, depth, B, T, D, theta);\n", "", 0),
    ("rope_bf16_truncates", "bits += 0x7fffu + lsb;", "(void)lsb;", 0),
    ("commit_copies_node_j", "* T + nodes[j]) * D;", "* T + j) * D;", 0),
    ("commit_v_from_k", "memcpy((char *)v_cache + dst * esz, (const char *)v_tree",
     "memcpy((char *)v_cache + dst * esz, (const char *)k_tree", 0),
    ("commit_length_short", "new_prefix_len[b] = ok ? P + L : P;",
     "new_prefix_len[b] = ok ? P + L - 1 : P;", 0),
    ("commit_ignores_tree_err", "int ok = !(tree_err && tree_err[b] != 0);", "int ok = 1;", 0),
    ("topk_ties_to_larger_token", "if (best < 0 || l > bl) {", "if (best < 0 || l >= bl) {", 0),
    ("topk_not_normalised", "(bl - m) - log(Z);", "(bl - m);", 0),
    ("topk_sum_not_shifted", "if (l > -INFINITY) Z += exp(l - m);",
     "if (l > -INFINITY) Z += exp(l);", 0),
    ("draft_key_not_cumulative", "ckey[npend] = cm[last] + klp[r];", "ckey[npend] = klp[r];", 0),
    ("draft_ties_to_later_offer", "ckey[q] > ckey[best]", "ckey[q] >= ckey[best]", 0),
    ("draft_row_of_parent", "topk_row(rows + (int64_t)last * V,",
     "topk_row(rows + (int64_t)(last ? par[last] : 0) * V,", 0),
    ("draft_level_off_by_one", "level[last] < max_levels", "level[last] <= max_levels", 0),
    ("draft_only_best_child", "for (int r = 0; r < K; ++r) {\n                    ckey",
     "for (int r = 0; r < 1; ++r) {\n                    ckey", 0),
    ("draft_token_of_parent", "tk[n] = ctok[best];", "tk[n] = tk[cpar[best]];", 0),
    ("draft_cum_in_f32", "cm[n] = ckey[best];", "cm[n] = (float)ckey[best];", 0),
    ("append_without_prefix_offset", "b, h, (int64_t)P + i);", "b, h, (int64_t)i);", 0),
    ("append_hides_refusal", "tree_err[b] = 3;", "tree_err[b] = 0;", 0),
    ("incache_tree_at_index", "num_blocks, b, kvh, P + j);", "num_blocks, b, kvh, j);", 0),
    ("compact_reads_destination", "(int64_t)P + nodes[j]);", "(int64_t)P + j);", 0),
    ("compact_length_short", "new_prefix_len[b] = ok ? P + L : P;",
     "new_prefix_len[b] = ok ? P + L - 1 : P;", 1),
    ("compact_ignores_tree_err", "int ok = !(tree_err && tree_err[b] != 0);", "int ok = 1;", 1),
    ("draft_prefers_last_parent", "if (!used[q] && (best < 0 || ckey[q] > ckey[best])) best = q;",
     "if (!used[q] && (best < 0 || ckey[q] > ckey[best] || (cpar[q] == last && cpar[best] != last))) best = q;", 0),
]


def _mutate(src: str, old: str, new: str, occ: int) -> str:
    assert src.count(old) >= occ + 1, f"mutation anchor not found: {old!r}"
    pos = -1
    for _ in range(occ + 1):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


_RUNNER = """
import sys
sys.path[:0] = [{tests!r}, {root!r}]
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except AssertionError:
        print("caught by", pin.__name__)
        sys.exit(3)
sys.exit(0)
"""


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ):
    src = open(SRC).read()
    tests = os.path.dirname(os.path.abspath(__file__))
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mutant.c")
        with open(path, "w") as f:
            f.write(_mutate(src, old, new, occ))
        lib = oracle.build(src=path, out=os.path.join(td, f"lib{name}.so"))
        code = _RUNNER.format(tests=tests, root=os.path.dirname(tests), lib=lib)
        # each mutant runs in its own process, under a time limit
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=120, env={**os.environ, "OMP_NUM_THREADS": "2"})
        assert r.returncode == 3, f"mutant {name} passed every pin (rc={r.returncode})\n{r.stderr[-2000:]}"
