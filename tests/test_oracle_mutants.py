"""Plant plausible mistakes in a copy of the oracle and show a pin catches each.

Each mutant is a one-token edit of oracle.c (a dropped term, a wrong sign,
index or bias, a transposed operand), compiled on the CPU into a temporary
library.  The real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_sm_scale": ("z[t] = sm_scale * acc;", "z[t] = acc;"),
    "exp_sign": ("z[t] = exp(z[t] - zmax);", "z[t] = exp(zmax - z[t]);"),
    "no_normalise": ("o[d] = acc / wsum;", "o[d] = acc;"),
    "page_slot_swapped": ("table[(int64_t)b * max_pages + t / page_size]",
                          "table[(int64_t)b * max_pages + t % page_size]"),
    "slot_dropped": ("int64_t slot = t % page_size;", "int64_t slot = 0;"),
    "head_mapping": ("int32_t h = g * group + hh;", "int32_t h = hh * Hkv + g;"),
    "kv_head_ignored": ("+ (int64_t)g * head_stride;", ";"),
    "e4m3_bias": ("mag = ldexp(1.0 + (double)m / 8.0, e - 7);",
                  "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal": ("mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    "e4m3_nan": ("if (e == 15 && m == 7) return NAN;", "if (e == 15 && m == 7) return 480.0;"),
    "f16_bias": ("mag = ldexp(1.0 + (double)m / 1024.0, e - 15);",
                 "mag = ldexp(1.0 + (double)m / 1024.0, e - 14);"),
    "v_scale_dropped": ("Vd[(int64_t)t * D + d] = kv_element(v_base, row + d, kv_dtype, v_scale);",
                        "Vd[(int64_t)t * D + d] = kv_element(v_base, row + d, kv_dtype, 1.0);"),
    "k_scale_dropped": ("Kd[(int64_t)t * D + d] = kv_element(k_base, row + d, kv_dtype, k_scale);",
                        "Kd[(int64_t)t * D + d] = kv_element(k_base, row + d, kv_dtype, 1.0);"),
    "k_v_swapped": ("Kd[(int64_t)t * D + d] = kv_element(k_base,",
                    "Kd[(int64_t)t * D + d] = kv_element(v_base,"),
    "last_token_dropped": ("for (int32_t t = 0; t < L; ++t) {\n      int64_t page",
                           "for (int32_t t = 0; t < L - 1; ++t) {\n      int64_t page"),
    "empty_not_inert": ("if (L <= 0) {\n      memset", "if (L < 0) {\n      memset"),
    "topk_ascending": ("if (x->key != y->key) return x->key > y->key ? -1 : 1;",
                       "if (x->key != y->key) return x->key < y->key ? -1 : 1;"),
    "topk_tie_order": ("return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);",
                       "return x->idx > y->idx ? -1 : (x->idx < y->idx ? 1 : 0);"),
    "topk_negative_key": ("return (u & 0x80000000u) ? ~u : (u | 0x80000000u);",
                          "return (u & 0x80000000u) ? u : (u | 0x80000000u);"),
    "topk_sign_flip_key": ("return (u & 0x80000000u) ? ~u : (u | 0x80000000u);",
                           "return u ^ 0x80000000u;"),
    "topk_n_valid_ignored": ("int32_t m = n_valid ? n_valid[r] : n_blocks;",
                             "int32_t m = n_blocks;"),
    "topk_one_short": ("int32_t t = m < k ? m : k;", "int32_t t = m < k ? m : k - 1;"),
    "topk_rank_order_out": ("qsort(o, (size_t)t, sizeof(int32_t), cmp_int);", ";"),
    "topk_no_clamp": ("if (m > n_blocks) m = n_blocks;", ";"),
    "page4_unsorted": ("qsort(ids, (size_t)n_full, sizeof(int32_t), cmp_int); /* locality order */",
                       ";"),
    "page4_sort_tail_too": ("qsort(ids, (size_t)n_full, sizeof(int32_t), cmp_int); /* locality",
                            "qsort(ids, (size_t)n_pages, sizeof(int32_t), cmp_int); /* locality"),
    "page4_views_ignored": ("ids[k] = p * vpages_per_page + (int32_t)",
                            "ids[k] = p * (page_size / 4) + (int32_t)"),
    "page4_group_index": ("(((int64_t)b * 4 % page_size) / 4)", "(((int64_t)b % page_size) / 4)"),
    "page4_tail_len": ("out_len[r] = 4 * n_full + n_tail;", "out_len[r] = 4 * n_full;"),
    "page4_causal_block": ("const int32_t c = (L - 1) / 4;", "const int32_t c = L / 4;"),
    "page4_partial_ok": ("if (below != 4 * n_full) status |= PAGE4_PARTIAL;", ";"),
    "page4_stale_kept": ("if (trow[i] >= 0 && trow[i] < L) set[m++] = trow[i];",
                         "if (trow[i] >= 0 && trow[i] <= L) set[m++] = trow[i];"),
    "page4_no_dedupe": ("if (u == 0 || set[i] != set[u - 1]) set[u++] = set[i];",
                        "set[u++] = set[i];"),
    "page4_tail_unchecked": ("if (n_tail > 0 && set[m - 1] != 4 * c + n_tail - 1) status |= PAGE4_TAIL;",
                             ";"),
    "page4_page_unchecked": ("if (p < 0 || p >= num_pages) {", "if (p < 0) {"),
    "page4_overflow_unchecked": ("if (n_pages > out_stride) status |= PAGE4_OVERFLOW;", ";"),
    "mask_norm_over_row": ("for (int32_t i = 0; i < n; ++i) W += exp((double)z[items[i].idx] - m);",
                           "for (int32_t i = 0; i < V; ++i) W += exp((double)z[items[i].idx] - m);"),
    "mask_mass_includes_self": ("before += exp((double)z[items[i - 1].idx] - m);",
                                "before += exp((double)z[items[i].idx] - m);"),
    "mask_k_ignored": ("const int32_t n = k < V ? k : V;", "const int32_t n = V;"),
    "mask_p_ignored": ("if (p < 1.0f) {", "if (0) {"),
    "mask_first_not_kept": ("      keep = 1;\n      for (int32_t i = 1; i < n; ++i) {",
                            "      keep = 0;\n      for (int32_t i = 1; i < n; ++i) {"),
    "mask_invalid_masked": ("for (int32_t t = 0; t < V; ++t) o[t] = z[t];",
                            "for (int32_t t = 0; t < V; ++t) o[t] = -INFINITY;"),
    "mask_k_bound": ("if (k < 1 || k > k_max) st |= MASK_BAD_K;",
                     "if (k < 1 || k >= k_max) st |= MASK_BAD_K;"),
    "mask_p_nan_unchecked": ("if (isnan(p)) st |= MASK_BAD_P;", ";"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                    "-ffp-contract=off", str(src), "-o", lib, "-lm"], check=True)
    # Run the pins in a child process: a mutant may also crash outright,
    # which counts as caught.
    script = (
        "import sys\n"
        "from tests import oracle_pins\n"
        "failed = []\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(sys.argv[1])\n"
        "    except Exception as e:\n"
        "        failed.append(pin.__name__)\n"
        "print('FAILED_PINS', failed)\n")
    res = subprocess.run([sys.executable, "-c", script, lib], cwd=ROOT,
                         capture_output=True, text=True, timeout=600)
    crashed = res.returncode < 0          # killed by a signal (e.g. SIGSEGV)
    failed_some = "FAILED_PINS [" in res.stdout and "FAILED_PINS []" not in res.stdout
    assert crashed or failed_some, (
        f"mutant {name} not caught: rc={res.returncode}\n{res.stdout}\n{res.stderr[-2000:]}")
    print(name, "crashed" if crashed else res.stdout.strip())
