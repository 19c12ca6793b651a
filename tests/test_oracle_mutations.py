"""The oracle's pins must catch a plausible mistake anywhere in it.

Each case below plants one mistake in a copy of the oracle's C source (a
flipped sign, a dropped or wrong term, a wrong index, tie rule or
comparison), compiles it with the oracle's own flags, loads it in place of the
oracle and runs the pins that cover that part: at least one of them must fail.
The committed oracle is never modified; the mutants live in a temporary
directory for the length of the test session.
"""
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle as O
import test_oracle_attn_kl as T_attn
import test_oracle_commit as T_commit
import test_oracle_cosine as T_cos
import test_oracle_formats as T_fmt
import test_oracle_kmeans as T_km
import test_oracle_topk_gather as T_tg

SRC = os.path.join(os.path.dirname(O.__file__), "polestar_oracle.c")
HDR = os.path.join(os.path.dirname(O.__file__), "polestar_oracle.h")

# name, text in the source (must occur exactly once), planted replacement,
# pins (test function, args) expected to notice; a mistake spanning several
# places gives tuples of texts and replacements
MUTATIONS = [
    ("e4m3 ties to odd", "(dist == bestd && (c & 1) == 0)", "(dist == bestd && (c & 1) == 1)",
     [(T_fmt.test_e4m3_encode_matches_torch_in_range_and_on_ties, ())]),
    ("e4m3 saturates one code low", "if (x >= 448.0f) return 0x7e;", "if (x >= 448.0f) return 0x7d;",
     [(T_fmt.test_e4m3_saturates_and_handles_nonpositive, ())]),
    ("e2m1 ties to odd", "(dist == bestd && (i & 1) == 0)", "(dist == bestd && (i & 1) == 1)",
     [(T_fmt.test_e2m1_golden_tie_table, ())]),
    ("e2m1 keeps -0", "if (best == 0) return 0;\n", "\n",
     [(T_fmt.test_e2m1_golden_tie_table, ()), (T_fmt.test_nvfp4_zero_residual_row, ())]),
    ("row scale 2048 instead of 6*448", "const float g = A / 2688.0f;", "const float g = A / 2048.0f;",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()),
      (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("block scale over 4 instead of 6", "float t = Ab / 6.0f;", "float t = Ab / 4.0f;",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()),
      (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("residual sign flipped", "r[e] = x - c[e];", "r[e] = c[e] - x;",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()),
      (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("rebuilt row not rescaled by the norm", "(c[e] + rhat) * n);", "(c[e] + rhat));",
     [(T_tg.test_gather_rebuilds_representable_rows_exactly, ())]),
    ("row norm not square-rooted", "return (float)sqrt(ss);\n}", "return (float)ss;\n}",
     [(T_km.test_row_norms_fp64_exact_on_small_integers, ())]),
    ("update sums the non-members", "if (aw[j] != k) continue;\n            ++cnt;",
     "if (aw[j] == k) continue;\n            ++cnt;",
     [(T_km.test_k1_is_normalised_mean, ()), (T_km.test_centres_are_unit_and_member_means, ())]),
    ("singleton clusters keep their centre", "if (cnt > 0 && nrm > 0.0)", "if (cnt > 1 && nrm > 0.0)",
     [(T_km.test_singleton_cluster_centre_is_its_row, ())]),
    ("assignment ties to the highest index", "if (k == 0 || dot > bests)", "if (k == 0 || dot >= bests)",
     [(T_km.test_converged_assignment_is_argmax, ()), (T_km.test_assignment_ties_go_to_lowest_index, ())]),
    ("assignment against unrounded centres",
     "return dtype == PSO_BF16 ? (double)pso_bf16_to_f32(pso_f32_to_bf16(c)) : (double)c;",
     "return (double)c;",
     [(T_km.test_assignment_uses_bf16_rounded_centres, ())]),
    ("keys divided by count + 1", "(float)(acc[i] / (double)nw[k])", "(float)(acc[i] / (double)(nw[k] + 1))",
     [(T_km.test_centroid_keys_are_member_means_bf16, ()), (T_km.test_k_equals_n_gives_rows_and_exact_keys, ())]),
    ("farthest-first picks the most similar row", "if (seed < 0 || m[j] < m[seed]) seed = j;",
     "if (seed < 0 || m[j] > m[seed]) seed = j;",
     [(T_km.test_farthest_seeds_hit_every_planted_direction, ())]),
    ("strided seeds off by one row", "int j = (int)(((int64_t)k * N) / K);",
     "int j = (int)(((int64_t)k * N) / K) + (k + 1 < K);",
     [(T_km.test_strided_init_rows, ())]),
    ("logits without the softmax scale", "z[k] = sigma * dot;", "z[k] = dot;",
     [(T_attn.test_k_equals_n_is_textbook_attention, (4, 4))]),
    ("query head h reads KV head h mod Hkv", "const int g = h / G;", "const int g = h % Hkv;",
     [(T_attn.test_gqa_equals_replicated_heads, ()), (T_attn.test_k_equals_n_is_textbook_attention, (6, 2))]),
    ("KL weighted by the previous distribution", "D += exp(l) * (l - lp);", "D += exp(lp) * (l - lp);",
     [(T_attn.test_kl_two_point_closed_form, ()), (T_attn.test_kl_direction_is_current_against_previous, ())]),
    ("per-token drift averaged over rows, not heads",
     "D_i[(size_t)w * Nb + i] = (float)(dacc[i] / (double)Hq);",
     "D_i[(size_t)w * Nb + i] = (float)(dacc[i] / (double)(Hq + 1));",
     [(T_attn.test_kl_matches_scipy_and_gibbs, ()), (T_attn.test_scores_decompose_the_drift, (O.SCORE_KL_SHARE,))]),
    ("share score drops the log ratio", "if (score_kind == PSO_SCORE_KL_SHARE)          sacc[k] += term;",
     "if (score_kind == PSO_SCORE_KL_SHARE)          sacc[k] += p;",
     [(T_attn.test_scores_decompose_the_drift, (O.SCORE_KL_SHARE,))]),
    ("top-k ties to the higher index", "return ia < ib;", "return ia > ib;",
     [(T_tg.test_topk_matches_brute_force, (s,)) for s in range(6)]),
    ("top-k ranks NaN first", "if (na != nb) return nb;", "if (na != nb) return na;",
     [(T_tg.test_topk_matches_brute_force, (s,)) for s in range(6)]),
    ("gather takes the unselected clusters", "if (a < 0 || a >= K || !sel[a]) continue;",
     "if (a < 0 || a >= K || sel[a]) continue;",
     [(T_tg.test_gather_matches_set_filter, ("ample",))]),
    ("cosine drift with the wrong sign", "score[wk] = (float)(1.0 - dot);", "score[wk] = (float)(1.0 + dot);",
     [(T_cos.test_identical_opposite_orthogonal_are_exact, ())]),
    ("commit threshold not strict", "drift_rule = dl > (double)alpha * (gap * gap);",
     "drift_rule = dl >= (double)alpha * (gap * gap);",
     [(T_commit.test_threshold_is_strict_and_confidence_is_inclusive, ())]),
    ("commit mean includes the current step", "const double mean = hist_sum[r] / (double)n;",
     "const double mean = (hist_sum[r] + D) / (double)(n + 1);",
     [(T_commit.test_worked_case_delta_against_earlier_mean, ())]),
    ("commit threshold with an unsquared gap", "dl > (double)alpha * (gap * gap)", "dl > (double)alpha * gap",
     [(T_commit.test_worked_case_delta_against_earlier_mean, ())]),
    ("confidence rule not inclusive", "const int conf_rule = c >= tau_s;", "const int conf_rule = c > tau_s;",
     [(T_commit.test_threshold_is_strict_and_confidence_is_inclusive, ())]),
    ("suffix cluster at exactly half", "2 * in_suffix[c] > members[c]", "2 * in_suffix[c] >= members[c]",
     [(T_commit.test_suffix_majority_is_strict_and_boundary_row_is_not_suffix, ())]),
    ("suffix starts one row early", "first = block_start + s->Nb;", "first = block_start + s->Nb - 1;",
     [(T_commit.test_suffix_majority_is_strict_and_boundary_row_is_not_suffix, ()),
      (T_commit.test_suffix_worked_case, ())]),
    ("bf16 conversion truncates", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0u;",
     [(T_fmt.test_bf16_rounding_matches_torch, ())]),
    ("bf16 conversion ties away from even", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;",
     [(T_fmt.test_bf16_rounding_matches_torch, ())]),
    ("e4m3 subnormal step 2^-8", "if (e == 0) v = ldexp((double)m, -9);", "if (e == 0) v = ldexp((double)m, -8);",
     [(T_fmt.test_e4m3_decode_all_codes_matches_torch, ())]),
    ("log-softmax without the log", "const double lse = zmax + log(se);", "const double lse = zmax + se;",
     [(T_attn.test_logp_normalised, ()), (T_attn.test_k_equals_n_is_textbook_attention, (4, 4))]),
    ("drift history keeps only the last drift", "hist_sum[r] = (n > 0 ? hist_sum[r] : 0.0) + D;",
     "hist_sum[r] = D;", [(T_commit.test_delta_is_drift_minus_numpy_mean_of_earlier_steps, ())]),
    ("cosine drift of a centre with itself", "const float* b = C_prev + wk * d;", "const float* b = C_cur + wk * d;",
     [(T_cos.test_identical_opposite_orthogonal_are_exact, ())]),
    ("abs score without the absolute value", "sacc[k] += fabs(term);", "sacc[k] += term;",
     [(T_attn.test_abs_score_bounds_share, ())]),
    ("attention-weighted score ignores the attention", "sacc[k] += p * D;", "sacc[k] += D;",
     [(T_attn.test_scores_decompose_the_drift, (O.SCORE_ATTN_WEIGHTED,))]),
    ("attention-weighted score by the previous step's attention", "sacc[k] += p * D;",
     "sacc[k] += exp(lp) * D;",
     [(T_attn.test_worked_case_attention_weighted_score, ())]),
    ("abs score as the absolute value of the summed terms",
     ("sacc[k] += fabs(term);",
      "score[(size_t)w * K + k] = (float)(sacc[k] / (double)Hq);"),
     ("sacc[k] += term;",
      "score[(size_t)w * K + k] = (float)((score_kind == PSO_SCORE_KL_SHARE_ABS ? fabs(sacc[k]) : sacc[k])"
      " / (double)Hq);"),
     [(T_attn.test_worked_case_share_and_abs_scores, ())]),
    ("top-k ranks the lowest scores first", "if (!na && a != b) return a > b;", "if (!na && a != b) return a < b;",
     [(T_tg.test_topk_matches_brute_force, (0,))]),
    ("unit rows by a rounded reciprocal", "return n > 0.0f ? h / n : 0.0f;", "return n > 0.0f ? h * (1.0f / n) : 0.0f;",
     [(T_km.test_strided_init_rows, ()), (T_km.test_k1_is_normalised_mean, ()),
      (T_km.test_centres_are_unit_and_member_means, ()), (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("centre divided by the member count instead of its norm", "(float)(S[e] / nrm);", "(float)(S[e] / cnt);",
     [(T_km.test_k1_is_normalised_mean, ()), (T_km.test_centres_are_unit_and_member_means, ())]),
    ("member rows weighted by their norm instead of its reciprocal", "const double inv = 1.0 / (double)rn[j];",
     "const double inv = (double)rn[j];",
     [(T_km.test_k1_is_normalised_mean, ()), (T_km.test_centres_are_unit_and_member_means, ())]),
    ("residual coded from h instead of h / n", "float x = unit_elem(ld(H, dtype, row * d + e), n);",
     "float x = ld(H, dtype, row * d + e);",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()), (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("gather lists the members in descending order",
     "        for (int j = 0; j < N; ++j) {\n            const size_t row = (size_t)w * N + j;\n"
     "            int a = assign[row];\n            if (a < 0 || a >= K || !sel[a]) continue;",
     "        for (int j = N - 1; j >= 0; --j) {\n            const size_t row = (size_t)w * N + j;\n"
     "            int a = assign[row];\n            if (a < 0 || a >= K || !sel[a]) continue;",
     [(T_tg.test_gather_matches_set_filter, ("ample",)), (T_tg.test_gather_matches_set_filter, ("short",))]),
    ("queries read head-major", "const size_t qo = (((size_t)w * Nb + i) * Hq + h) * dh;",
     "const size_t qo = (((size_t)w * Hq + h) * Nb + i) * dh;",
     [(T_attn.test_k_equals_n_is_textbook_attention, (4, 4)), (T_attn.test_k_equals_n_is_textbook_attention, (6, 2))]),
    ("log-sum-exp without the max shift", "const double lse = zmax + log(se);", "const double lse = log(se);",
     [(T_attn.test_logp_normalised, ()), (T_attn.test_k_equals_n_is_textbook_attention, (4, 4))]),
    ("block scale from the first half of the block",
     "for (int e = 16 * b; e < 16 * b + 16; ++e)\n                    if (fabsf(r[e]) > Ab) Ab = fabsf(r[e]);",
     "for (int e = 16 * b; e < 16 * b + 8; ++e)\n                    if (fabsf(r[e]) > Ab) Ab = fabsf(r[e]);",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()), (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("code nibbles swapped", "cr[e / 2] = (uint8_t)(lo | (hi << 4));", "cr[e / 2] = (uint8_t)(hi | (lo << 4));",
     [(T_fmt.test_nvfp4_round_trip_exact_on_representable_rows, ()), (T_fmt.test_nvfp4_error_bound_random_rows, ())]),
    ("row norm skips the last element",
     "    for (int e = 0; e < d; ++e) {\n        double h = (double)ld(H, dtype, row_off + (size_t)e);",
     "    for (int e = 0; e < d - 1; ++e) {\n        double h = (double)ld(H, dtype, row_off + (size_t)e);",
     [(T_km.test_row_norms_fp64_exact_on_small_integers, ())]),
]


def _compile(args):
    name, src, out = args
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-Wno-unused-variable",
           "-Wno-unused-but-set-variable", "-Wno-unused-parameter", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", src, "-o", out, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return name, r.returncode, r.stderr


@pytest.fixture(scope="module")
def mutants():
    base = open(SRC).read()
    tmp = tempfile.TemporaryDirectory(prefix="pso_mutants_")
    hdr = open(HDR).read()
    jobs = []
    for i, (name, old, new, _) in enumerate(MUTATIONS):
        # one mistake may need edits in several places: tuples of texts
        olds, news = (old, new) if isinstance(old, tuple) else ((old,), (new,))
        src = base
        for o, n in zip(olds, news):
            assert base.count(o) == 1, f"mutation {name!r}: target text occurs {base.count(o)} times"
            src = src.replace(o, n)
        d = os.path.join(tmp.name, f"m{i}")
        os.makedirs(d)
        open(os.path.join(d, "polestar_oracle.h"), "w").write(hdr)
        open(os.path.join(d, "polestar_oracle.c"), "w").write(src)
        jobs.append((name, os.path.join(d, "polestar_oracle.c"), os.path.join(d, "libmutant.so")))
    with ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(_compile, jobs))
    for name, rc, err in results:
        assert rc == 0, f"mutant {name!r} does not compile:\n{err}"
    yield {name: out for (name, _, out) in jobs}
    tmp.cleanup()


class _Swapped:
    """Load a mutant library in place of the oracle's for the duration."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        self.saved = (O._build.LIB, O._lib)
        O._build.LIB, O._lib = self.path, None

    def __exit__(self, *exc):
        O._build.LIB, O._lib = self.saved
        return False


def test_pins_pass_on_the_oracle_itself():
    for _, _, _, pins in MUTATIONS:
        for fn, args in pins:
            fn(*args)


@pytest.mark.parametrize("idx", range(len(MUTATIONS)), ids=[m[0] for m in MUTATIONS])
def test_pins_catch_a_planted_mistake(mutants, idx):
    name, _, _, pins = MUTATIONS[idx]
    caught = []
    with _Swapped(mutants[name]):
        for fn, args in pins:
            try:
                fn(*args)
            except Exception as e:  # an assertion, or an error the mutant raises
                caught.append(f"{fn.__name__}: {type(e).__name__}")
    assert caught, f"no pin noticed the planted mistake {name!r}"
