"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/tes_oracle.cpp, changes one expression into a
plausible mistake (a flipped tie rule, a floor turned into rounding, an
off-by-one in the top-p test, a swapped Philox word, ...), builds the copy
into a temporary directory and runs the pin battery against it.  The test
passes only if at least one pin fails for every planted mistake.  Nothing
here touches the GPU.
"""

import os
import subprocess

import pytest

import oracle
import tests.test_oracle_brute as pb
import tests.test_oracle_logits as pl
import tests.test_oracle_spec as ps_
import tests.test_oracle_philox as pp
import tests.test_oracle_properties as pr

SRC = os.path.join(os.path.dirname(oracle.__file__), "tes_oracle.cpp")

MUTATIONS = {
    "tie_to_higher_index": (
        "return key[a] > key[b]; });",
        "return key[a] != key[b] ? key[a] > key[b] : a > b; });"),
    "negatives_not_sanitised": (
        "if (std::isnan(x) || std::signbit(x)) return 0u;",
        "if (std::isnan(x)) return 0u;"),
    "mass_rounds_instead_of_floor": (
        "return (uint64_t)std::floor(std::ldexp(v, 32));",
        "return (uint64_t)std::nearbyint(std::ldexp(v, 32));"),
    "mass_not_saturated": (
        "if (v >= 1.0) return (uint64_t)1 << 32;",
        "if (v >= 2.0) return (uint64_t)1 << 33;"),
    "threshold_floor_not_ceil": (
        "(((uint64_t)prod & 0xFFFFFFu) != 0 ? 1 : 0)",
        "0"),
    "keep_while_not_strict": (
        "while (kept < k_eff && s_excl < T)",
        "while (kept < k_eff && s_excl <= T)"),
    "draw_compare_not_strict": (
        "while (s_incl <= t)",
        "while (s_incl < t)"),
    "uniform_words_swapped": (
        "return (uint64_t)out[0] | ((uint64_t)out[1] << 32);",
        "return (uint64_t)out[1] | ((uint64_t)out[0] << 32);"),
    "philox_weyl_constant": (
        "kPhiloxWeyl1 = 0xBB67AE85u;",
        "kPhiloxWeyl1 = 0xBB67AE86u;"),
    "philox_key_word": (
        "uint32_t n0 = hi1 ^ c[1] ^ k[0];",
        "uint32_t n0 = hi1 ^ c[1] ^ k[1];"),
    "counter_row_offset_swapped": (
        "uint32_t ctr[4] = {(uint32_t)offset, (uint32_t)(offset >> 32), (uint32_t)row,\n"
        "                       (uint32_t)(row >> 32)};",
        "uint32_t ctr[4] = {(uint32_t)row, (uint32_t)(row >> 32), (uint32_t)offset,\n"
        "                       (uint32_t)(offset >> 32)};"),
    "p_truncated": (
        "double r = std::nearbyint(scaled);",
        "double r = std::floor(scaled);"),
    "p_not_clamped_low": (
        "if (!(p > 0.0f)) return 1;",
        "if (!(p > 0.0f)) return 0;"),
    "inf_draw_modulo": (
        "uint64_t t = (uint64_t)(((u128)u * (u128)inf_count) >> 64);",
        "uint64_t t = u % (uint64_t)inf_count;"),
    "inf_weight": (
        "float w = (float)(1.0 / (double)inf_count);",
        "float w = (float)(1.0 / (double)(inf_count + 1));"),
    "zero_mass_first_sorted": (
        "*token = (int32_t)*std::min_element(order.begin(), order.end());",
        "*token = (int32_t)order[0];"),
    "min_p_floor_not_ceil": (
        "return (uint64_t)q + (rem ? 1 : 0);",
        "return (uint64_t)q;"),
    "min_p_strict": (
        "q[n_min_p] >= floor_mass",
        "q[n_min_p] > floor_mass"),
    "min_p_from_last_support_mass": (
        "min_p_floor_mass(theta, q[0])",
        "min_p_floor_mass(theta, q[k_eff - 1])"),
    "min_p_cut_dropped": (
        "if (n_min_p < kept) {",
        "if (n_min_p > kept) {"),
    "temperature_multiplies": (
        "else r = (float)(1.0 / (double)tau);",
        "else r = tau;"),
    "tau_zero_not_the_limit": (
        "if (!(tau > 0.0f)) r = std::numeric_limits<float>::infinity();",
        "if (!(tau > 0.0f)) r = 1.0f;"),
    "exp_low_part_dropped": (
        "f = std::fma(n, -ln2_lo, f);",
        "f = f + 0.0f;"),
    "exp_taylor_degree_six": (
        "float p = taylor_coefficient(7);",
        "float p = 0.0f;"),
    "logit_nan_counts_as_max": (
        "const float xi = std::isnan(x[i]) ? ninf : x[i];\n        if (xi > M) M = xi;",
        "const float xi = std::isnan(x[i]) ? -ninf : x[i];\n        if (xi > M) M = xi;"),
    "spec_accept_strict": (
        "return hi < rhs || (hi == rhs && low == 0);",
        "return hi < rhs;"),
    "spec_residual_sign_swapped": (
        "r[x] = a > b ? a - b : 0;",
        "r[x] = b > a ? b - a : 0;"),
    "spec_acceptance_uses_draw_words": (
        "const uint64_t ua = oracle_uniform_u64_hi(seed, (uint64_t)g, offset);",
        "const uint64_t ua = oracle_uniform_u64(seed, (uint64_t)g, offset);"),
    "spec_map_ignored": (
        "return target_map ? (int64_t)target_map[n * (L + 1) + l] : l;",
        "return (int64_t)l;"),
    "spec_zero_residual_gives_minus_one": (
        "int32_t corr = tok;",
        "int32_t corr = -1;"),
    "spec_correction_draws_with_acceptance_uniform": (
        "const u128 t = (u128)u * R_hi + (((u128)u * R_lo) >> 64);",
        "const u128 t = (u128)ua * R_hi + (((u128)ua * R_lo) >> 64);"),
    "spec_draft_mass_not_sanitised": (
        "const uint64_t Qd = fixed_point_mass(sanitized_key(y[d]));",
        "const uint64_t Qd = fixed_point_mass(sanitized_key(std::fabs(y[d])));"),
    "renorm_by_topk_mass": (
        "renorm[order[j]] = (float)((double)q[j] / (double)M_p);",
        "renorm[order[j]] = (float)((double)q[j] / (double)M_k);"),
}


def _pins(orc, torch_exe, rocrand_exe):
    """Yield callables; each raises AssertionError when a pin fails."""
    yield lambda: pb.test_exact_p_boundaries(orc)
    yield lambda: pb.test_p_rounds_half_to_even(orc)
    yield lambda: pb.test_heavy_ties(orc)
    for V in (1, 3, 8):
        yield lambda V=V: pb.test_plain_and_special_rows(orc, V)
    yield lambda: pb.test_rows_with_infinities(orc, 4)
    yield lambda: pr.test_zero_mass_rows_return_smallest_support_index(orc)
    yield lambda: pr.test_masses_closed_form(orc)
    yield lambda: pr.test_equal_values_keep_ceil_pn(orc, 100, 0.77)
    yield lambda: pl.test_exp_weight_within_one_ulp(orc)
    yield lambda: pl.test_exp_weight_special_values(orc)
    yield lambda: pl.test_logit_weights_against_float64_softmax(orc)
    yield lambda: pl.test_logit_weight_rules(orc)
    for theta in (0.2, 0.25, 0.5, 1.0):
        yield lambda theta=theta: pl.test_min_p_against_brute_force(orc, theta)
    yield lambda: pl.test_min_p_floor_exactly_on_a_mass(orc)
    for special in (False, True):
        for use_map in (False, True):
            yield lambda a=special, b=use_map: ps_.test_spec_verify_against_brute_force(orc, a, b)
    yield lambda: ps_.test_acceptance_boundary(orc)
    yield lambda: ps_.test_identical_distributions_accept_everything(orc)
    if torch_exe:
        yield lambda: pp.test_block_function_matches_pytorch(orc, torch_exe)
        yield lambda: pp.test_row_uniform_mapping(orc, torch_exe)
    if rocrand_exe:
        yield lambda: pp.test_block_function_matches_rocrand(orc, rocrand_exe)


@pytest.fixture(scope="module")
def harnesses(tmp_path_factory):
    t = r = None
    try:
        t = pp._build(tmp_path_factory, "USE_TORCH", [pp.TORCH_INC])
    except BaseException:
        pass
    try:
        r = pp._build(tmp_path_factory, "USE_ROCRAND", [pp.ROCM_INC], ["__HIP_PLATFORM_AMD__"])
    except BaseException:
        pass
    return t, r


def test_unmutated_oracle_passes_every_pin(orc, harnesses):
    for pin in _pins(orc, *harnesses):
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, harnesses, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + name
    mutated = tmp_path / "tes_oracle_mut.cpp"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-ffp-contract=off", "-shared", "-fPIC",
                    "-pthread", "-o", str(lib), str(mutated)], check=True)
    mut = oracle.load(str(lib))
    for pin in _pins(mut, *harnesses):
        try:
            pin()
        except AssertionError:
            return
    pytest.fail("no pin caught the planted mistake " + name)
