"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong index or sign, a wrong
order, a wrong constant) in a copy of the oracle's C source, builds it on the
CPU, swaps it in, and runs the pin tests of test_oracle_layout.py and
test_oracle_numerics.py against it: at least one pin must fail. The planted
copy lives in a temporary directory and never leaves this test. Every planted
mistake keeps the oracle's memory accesses in bounds, so the pins (not a
crash) must be what catches it.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_groups as TG
from tests import test_oracle_layout as TL
from tests import test_oracle_numerics as TN
from tests import test_oracle_relay as TRL
from tests import test_oracle_swaps as TSW

SRC = os.path.join(os.path.dirname(oracle.__file__), "epx_oracle.c")

# (name, exact text in the source, replacement)
MUTANTS = [
    ("slot order j-major",
     "    for (int32_t t = 0; t < T; ++t)\n        for (int32_t j = 0; j < k; ++j) {\n            int32_t e = idx[(int64_t)t * k + j];\n            int32_t row = next[e];",
     "    for (int32_t j = 0; j < k; ++j)\n        for (int32_t t = 0; t < T; ++t) {\n            int32_t e = idx[(int64_t)t * k + j];\n            int32_t row = next[e];"),
    ("rank offset indexed by rank, not by its first expert",
     "        rank_offset[r] = expert_offset[r * epr];",
     "        rank_offset[r] = expert_offset[r];"),
    ("interleaved expert-to-rank map",
     "        for (int32_t e = r * epr; e < (r + 1) * epr; ++e)\n            rank_rows[r] += expert_count[e];",
     "        for (int32_t e = r; e < E; e += R)\n            rank_rows[r] += expert_count[e];"),
    ("rank tokens count duplicates",
     "                if (rank_of(idx[(int64_t)t * k + j], epr) == r)\n                    hit = 1;",
     "                if (rank_of(idx[(int64_t)t * k + j], epr) == r)\n                    hit += 1;"),
    ("host of an expert is its rank",
     "    return rank_of(e, epr) / rph;",
     "    return rank_of(e, epr) + 0 * rph;"),
    ("rank of an expert interleaved",
     "    return e / epr;",
     "    return e % (epr == 1 ? 1 << 30 : epr);"),
    ("own host left out of the relay rows",
     "                if (!hit) {\n                    relay_slot[(int64_t)t * H + h] = -1;",
     "                if (!hit || h == s / rph) {\n                    relay_slot[(int64_t)t * H + h] = -1;"),
    ("relay destination uses the host count",
     "        relay_dst_rank[h] = h * rph + (s % rph);",
     "        relay_dst_rank[h] = h * rph + (s % H);"),
    ("fan-out mask uses the expert id",
     "                        mask |= 1u << (rank_of(e, epr) % rph);",
     "                        mask |= 1u << (e % rph);"),
    ("fp8 scale constant",
     "            float s = a / 448.0f;",
     "            float s = a / 447.0f;"),
    ("fp8 quotient as x times 448/amax",
     "                    q[c] = oracle_f32_to_e4m3(v / s);",
     "                    q[c] = oracle_f32_to_e4m3(v * (448.0f / a));"),
    ("fp8 quotient as x times the reciprocal of the scale",
     "                    q[c] = oracle_f32_to_e4m3(v / s);",
     "                    q[c] = oracle_f32_to_e4m3(v * (1.0f / s));"),
    ("fp8 scale as amax times 1/448",
     "            float s = a / 448.0f;",
     "            float s = a * (1.0f / 448.0f);"),
    ("fp8 amax without abs",
     "                if (fabsf(v) > a)\n                    a = fabsf(v);",
     "                if (v > a)\n                    a = v;"),
    ("zero block drops the sign",
     "                    q[c] = signbit(v) ? 0x80 : 0x00;   /* all-zero block keeps the sign */",
     "                    q[c] = 0x00;"),
    ("e4m3 truncates the mantissa",
     "    float m = rintf((2.0f * f - 1.0f) * 8.0f); /* exact operands; half to even */",
     "    float m = floorf((2.0f * f - 1.0f) * 8.0f);"),
    ("e4m3 saturates too late",
     "    if (a >= 448.0f)\n        return (uint8_t)(sign | 0x7E);",
     "    if (a >= 480.0f)\n        return (uint8_t)(sign | 0x7E);"),
    ("e4m3 subnormal boundary",
     "    if (a < 0.015625f) {",
     "    if (a < 0.0078125f) {"),
    ("e4m3 exponent bias",
     "    int biased = unb + 7;",
     "    int biased = unb + 8;"),
    ("bf16 ties away from zero",
     "        pick_hi = (lo_bits >> 16) & 1u;           /* tie: keep the even one */",
     "        pick_hi = 1;"),
    ("combine drops the last expert",
     "            for (int32_t j = 0; j < k; ++j) {\n                int32_t row = slot[(int64_t)t * k + j];",
     "            for (int32_t j = 0; j + 1 < k; ++j) {\n                int32_t row = slot[(int64_t)t * k + j];"),
    ("combine transposes the weights",
     "                acc = fmaf(w[(int64_t)t * k + j], v, acc);",
     "                acc = fmaf(w[((int64_t)j * T + t) % ((int64_t)T * k)], v, acc);"),
    ("fan-out compares the rank with the host",
     "                if (host_of(e, epr, rph) != h)\n                    continue;\n                int64_t dst",
     "                if (rank_of(e, epr) != h)\n                    continue;\n                int64_t dst"),
    ("partials drop the last expert",
     "                for (int32_t j = 0; j < k; ++j) {\n                    int32_t e = idx[(int64_t)t * k + j];\n                    if (host_of(e, epr, rph) != h)",
     "                for (int32_t j = 0; j + 1 < k; ++j) {\n                    int32_t e = idx[(int64_t)t * k + j];\n                    if (host_of(e, epr, rph) != h)"),
    ("partials take the next weight",
     "                    acc = fmaf(w[(int64_t)t * k + j], oracle_bf16_to_f32(y[(int64_t)row * hidden + c]),",
     "                    acc = fmaf(w[(int64_t)t * k + (j + 1) % k], oracle_bf16_to_f32(y[(int64_t)row * hidden + c]),"),
    ("finish reads the first host only",
     "                int32_t r = relay_slot[(int64_t)t * H + h];\n                if (r < 0)\n                    continue;\n                float p",
     "                int32_t r = relay_slot[(int64_t)t * H];\n                if (r < 0)\n                    continue;\n                float p"),
    ("swap pairs heaviest with the second lightest",
     "            int32_t A = order[p], B = order[rph - 1 - p];",
     "            int32_t A = order[p], B = order[rph - 2 - p < p ? rph - 1 - p : rph - 2 - p];"),
    ("swap ties keep the last candidate",
     "                    if (best < 0 || m < best) {   /* strict: the first (a, b) keeps ties */",
     "                    if (best < 0 || m <= best) {"),
    ("swap ignores the threshold",
     "            int32_t applied = (old_max - best > 0) && (old_max - best >= tau);",
     "            int32_t applied = (old_max - best > 0);"),
    ("unplanned host reports load 0",
     "        if (host_bad[r / rph] != 0) {\n            load_before[r] = -1;",
     "        if (host_bad[r / rph] != 0) {\n            load_before[r] = 0;"),
    ("swap sorts lightest first",
     "                if (load_before[q] > load_before[r] || (load_before[q] == load_before[r] && q < r))",
     "                if (load_before[q] < load_before[r] || (load_before[q] == load_before[r] && q < r))"),
    ("groups interleave the local experts",
     "    return (e % epr) / (epr / m);",
     "    return (e % epr) % m;"),
    ("grouped rows j-major",
     "    for (int32_t t = 0; t < T; ++t)\n        for (int32_t j = 0; j < k; ++j) {\n            int32_t e = idx[(int64_t)t * k + j];\n            slot[(int64_t)t * k + j] = next[e];",
     "    for (int32_t j = 0; j < k; ++j)\n        for (int32_t t = 0; t < T; ++t) {\n            int32_t e = idx[(int64_t)t * k + j];\n            slot[(int64_t)t * k + j] = next[e];"),
    ("grouped offsets rank-major",
     "    for (int32_t g = 0; g < m; ++g)\n        for (int32_t r = 0; r < R; ++r) {\n            group_offset[g * R + r] = run;",
     "    for (int32_t r = 0; r < R; ++r)\n        for (int32_t g = 0; g < m; ++g) {\n            group_offset[g * R + r] = run;"),
    ("grouped combine takes the groups last to first",
     "            for (int32_t g = 0; g < m; ++g)\n                for (int32_t j = 0; j < k; ++j) {\n                    if (group_of",
     "            for (int32_t g = m - 1; g >= 0; --g)\n                for (int32_t j = 0; j < k; ++j) {\n                    if (group_of"),
    ("grouped combine in plain j order",
     "                    if (group_of(idx[(int64_t)t * k + j], epr, m) != g)\n                        continue;",
     "                    if (g != 0)\n                        continue;"),
    ("grouped combine subtracts",
     "                    acc = fmaf(wt, v, acc);",
     "                    acc = fmaf(-wt, v, acc);"),
    ("group slots keep later groups",
     "        slot_g[p] = group_of(idx[p], epr, m) == g ? slot[p] : -1;",
     "        slot_g[p] = group_of(idx[p], epr, m) >= g ? slot[p] : -1;"),
    ("combine subtracts",
     "                acc = fmaf(w[(int64_t)t * k + j], v, acc);",
     "                acc = fmaf(-w[(int64_t)t * k + j], v, acc);"),
]


def _pins():
    """The pin tests, as zero-argument callables."""
    calls = []
    for shape in TL.SMALL_SHAPES:
        for relay in (False, True):
            calls.append(lambda s=shape, r=relay: TL.test_layout_matches_brute_force(s, r))
    for case in ("one_expert", "duplicates", "random_with_dups"):
        calls.append(lambda c=case: TL.test_layout_degenerate_routing(c))
    calls.append(lambda: TL.test_copy_counts_monte_carlo(256, 8, 32, 4))
    calls.append(TL.test_rank_imbalance_worked_example)
    calls.append(TL.test_imbalance_ratio_constructed)
    calls.append(TN.test_e4m3_critical_points)
    calls.append(TN.test_e4m3_sign_symmetry_and_negative_sample)
    calls.append(TN.test_e4m3_decode_all_codes_vs_torch)
    calls.append(TN.test_bf16_rounding_vs_torch)
    calls.append(lambda: TN.test_fp8_block_properties(False))
    calls.append(lambda: TN.test_fp8_block_properties(True))
    calls.append(TN.test_fp8_quotient_golden_blocks)
    calls.append(lambda: TN.test_dispatch_bf16_rows_are_token_rows(False))
    calls.append(lambda: TN.test_dispatch_bf16_rows_are_token_rows(True))
    calls.append(TN.test_combine_within_float32_bound_of_float64_sum)
    calls.append(TN.test_combine_exact_special_cases)
    calls.append(TN.test_combine_identity_experts_return_x)
    calls.append(TN.test_combine_config_rule_closed_form)
    for shape in TRL.SHAPES:
        calls.append(lambda sh=shape: TRL.test_fanout_of_tagged_rows_brute_force(sh))
        calls.append(lambda sh=shape: TRL.test_partial_membership_exact(sh))
    calls.append(lambda: TRL.test_fanout_of_relay_dispatch_is_per_expert_dispatch(TRL.SHAPES[1]))
    calls.append(lambda: TRL.test_one_host_two_level_is_flat(8, 256, 32))
    calls.append(lambda: TRL.test_two_level_within_bounds_of_float64(TRL.SHAPES[1]))
    for shape in TG.SHAPES:
        calls.append(lambda sh=shape: TG.test_grouped_layout_brute_force(sh, False))
        calls.append(lambda sh=shape: TG.test_group_dispatches_cover_every_row_once(sh))
    calls.append(TG.test_combine_order_cases)
    calls.append(lambda: TG.test_one_group_is_the_plain_layout_and_combine((30, 4, 16, 4, 1)))
    calls.append(TSW.test_figure_example)
    for case in TSW.CASES:
        calls.append(lambda c=case: TSW.test_swaps_optimal_and_consistent(c, 5))
    calls.append(TSW.test_degenerate_cases)
    calls.append(TSW.test_bad_slot_ids_leave_only_their_host_unplanned)
    return calls


def _count_failures(lib):
    saved = oracle._lib
    oracle._lib = lib
    failed = 0
    try:
        for pin in _pins():
            try:
                pin()
            except (AssertionError, oracle.OracleError, ValueError, IndexError):
                failed += 1
    finally:
        oracle._lib = saved
    return failed


def test_unmodified_oracle_passes_every_pin():
    assert _count_failures(oracle.load()) == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique for {name!r}"
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        path = os.path.join(tmp, "epx_oracle.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", *oracle._CFLAGS, "-o", so, path, "-lm"], check=True)
        lib = oracle.load(so)
        assert _count_failures(lib) > 0, f"no pin caught the planted mistake {name!r}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
