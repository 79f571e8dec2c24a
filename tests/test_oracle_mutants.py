"""The pins must catch plausible mistakes in the oracle.

Each mutant below is a one-line change to a copy of the oracle's C++ source
(a dropped term, a wrong index or sign, a flipped tie-break, an off-by-one
window). The copy is built with g++ in a temporary directory, the pin tests
are re-run against it in a child process, and at least one of them must
fail (a mutant that crashes the child, e.g. by writing past a buffer, counts
as caught). Everything runs on the CPU."""

import os
import subprocess
import sys

import pytest

import oracle
from tests import test_oracle_append as Ap
from tests import test_oracle_attention as A
from tests import test_oracle_selection as S
from tests import test_oracle_widen as Wd

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvsp_oracle.cpp")

MUTANTS = {
    "head map h % Hkv": ("const int32_t g = h / G;", "const int32_t g = h % Hkv;"),
    "summary not divided by P": ("s[d] = sum / static_cast<double>(P);", "s[d] = sum;"),
    "summary over P-1 tokens": ("for (int32_t t = 0; t < P; ++t) sum +=",
                                "for (int32_t t = 1; t < P; ++t) sum +="),
    "ties to higher index": ("return score[a] > score[b]; });",
                             "return score[a] > score[b] || (score[a] == score[b] && a > b); });"),
    "score sign flipped": ("total += dot;", "total -= dot;"),
    "window rounded up": ("const int64_t C = hist / P;", "const int64_t C = ceil_div(hist, P);"),
    "ratio floored": ("k_req = ceil_div(C * keep_num, keep_den);",
                      "k_req = C * keep_num / keep_den;"),
    "floor ignored": ("int64_t k_eff = std::max<int64_t>(k_req, keep_floor);",
                      "int64_t k_eff = k_req;"),
    "gamma not strict": ("k_eff * static_cast<int64_t>(gamma_den) > static_cast<int64_t>(gamma_num) * C",
                         "k_eff * static_cast<int64_t>(gamma_den) >= static_cast<int64_t>(gamma_num) * C"),
    "merge without rescale": ("const double w = std::exp(m[i] - M);", "const double w = 1.0;"),
    "merge lse drops max": ("*lse = M + std::log(Lsum);", "*lse = std::log(Lsum);"),
    "values read from K": ("acc[d] += w * load_elem(dtype, v_pool,", "acc[d] += w * load_elem(dtype, k_pool,"),
    "window skips a block": ("for (int32_t t = C * P; t < L; ++t) tokens[count++] = t;",
                             "for (int32_t t = C * P + P; t < L; ++t) tokens[count++] = t;"),
    "spans never merge": ("ids[e] == ids[e - 1] + 1", "ids[e] == ids[e - 1]"),
    "token offset from wrong block": ("pool_index(phys, g, t % P, d, Hkv, P, D));\n    z[i]",
                                      "pool_index(phys, g, (t + 1) % P, d, Hkv, P, D));\n    z[i]"),
    "fp16 subnormal scale": ("std::ldexp(static_cast<double>(frac), -24)",
                             "std::ldexp(static_cast<double>(frac), -25)"),
    "default scale 1/D": ("scale = 1.0 / std::sqrt(static_cast<double>(D));",
                          "scale = 1.0 / static_cast<double>(D);"),
    "append one token late": ("const int64_t dst = pool_index(phys, g, t, 0, Hkv, P, D);",
                              "const int64_t dst = pool_index(phys, g, (t + 1) % P, 0, Hkv, P, D);"),
    "append value into K": ("std::memcpy(static_cast<char*>(v_pool) + dst * elem,\n                  static_cast<const char*>(v_new)",
                             "std::memcpy(static_cast<char*>(k_pool) + dst * elem,\n                  static_cast<const char*>(v_new)"),
    "append summary one token early": ("    if (t == P - 1) {\n      flags[b] = 1;",
                                       "    if (t == P - 2) {\n      flags[b] = 1;"),
    "append ignores table": ("const int32_t phys = block_table[static_cast<int64_t>(b) * max_blocks + j];\n    for (int32_t g = 0; g < Hkv; ++g) {\n      const int64_t src",
                             "const int32_t phys = j;\n    for (int32_t g = 0; g < Hkv; ++g) {\n      const int64_t src"),
}


def _pins():
    """Every pin, as (name, zero-argument callable)."""
    out = []
    for row in S.PLAN_TABLE:
        out.append((f"plan {row[0]}", lambda row=row: S.test_plan_table(row)))
    for P in (1, 4, 16):
        out.append((f"summary P={P}", lambda P=P: S.test_summary_closed_form(P)))
    out.append(("summary table", S.test_summaries_follow_block_table_and_skip_partial_blocks))
    for hq, hkv in ((4, 4), (8, 2), (6, 2), (12, 1)):
        out.append((f"score {hq}/{hkv}",
                    lambda a=hq, b=hkv: S.test_score_equals_block_mean_of_head_summed_logits(a, b)))
    out.append(("zero query", S.test_zero_query_scores_zero_and_selects_lowest_indices))
    out.append(("duplicate block", S.test_duplicate_block_tie_goes_to_lower_index))
    for seed in range(6):
        out.append((f"topk enum {seed}", lambda s=seed: S.test_topk_matches_subset_enumeration(s)))
    out.append(("topk sort", S.test_topk_matches_sort_by_key))
    out.append(("spans hand", S.test_spans_hand_example))
    out.append(("spans random", S.test_spans_invariants_random))
    out.append(("attended tokens", S.test_attended_tokens_sparse_and_dense))
    out.append(("fp16 widen", Wd.test_fp16_all_patterns_match_numpy))
    out.append(("bf16 widen", Wd.test_bf16_all_patterns_match_binary32_top_half))
    for args in (("fp32", 8, 8, 16, 1024, 32), ("fp16", 4, 2, 16, 333, 40),
                 ("bf16", 6, 2, 64, 640, 0)):
        out.append((f"full keep {args[0]}",
                    lambda a=args: A.test_full_keep_equals_textbook_dense(*a)))
    out.append(("dense fallback", A.test_dense_fallback_equals_textbook_dense))
    for seed in range(2):
        out.append((f"lse merge {seed}", lambda s=seed: A.test_lse_merge_partition_invariance(s)))
    out.append(("single token", A.test_single_token_gives_value_exactly))
    out.append(("equal logits", A.test_equal_logits_give_mean_of_values))
    out.append(("append fill", Ap.test_filling_a_block_token_by_token))
    out.append(("append fp16/fp32", Ap.test_filling_a_block_fp16_and_fp32))
    out.append(("append skip", Ap.test_negative_position_writes_nothing))
    out.append(("append batch", Ap.test_batch_append_lands_in_each_sequences_block_and_matches_summaries))
    return out


def _failing_pins(lib_path):
    prev = oracle.use_library(lib_path)
    failed = []
    try:
        for name, fn in _pins():
            try:
                fn()
            except (AssertionError, ValueError, IndexError):
                failed.append(name)
    finally:
        oracle.restore_library(prev)
    return failed


def test_unmodified_oracle_passes_every_pin(tmp_path):
    lib_path = oracle.build(src=SRC, out=str(tmp_path / "liboracle_copy.so"))
    assert _failing_pins(lib_path) == []


_CHILD = """
import sys
sys.path.insert(0, {root!r})
from tests.test_oracle_mutants import _failing_pins
failed = _failing_pins({lib!r})
print("failing pins:", failed)
sys.exit(0 if failed else 3)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(before) == 1, f"mutation site for {name!r} not unique"
    src = tmp_path / "kvsp_oracle_mutant.cpp"
    src.write_text(text.replace(before, after))
    lib_path = oracle.build(src=str(src), out=str(tmp_path / "libkvsp_oracle_mutant.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=root, lib=lib_path)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 3, f"no pin catches mutant {name!r}"
