"""Plants plausible mistakes in a copy of the oracle (CPU only) and checks
that the pins catch every one: a dropped or sign-flipped residual, swapped
K/V bases, a wrong query-to-KV-head map, a missing softmax scale, an
off-by-one rank, a transposed basis, a missing normalisation, a wrong
exponential base, and in the encoder a wrong tie rule, a wrong rounding
rule, a residual against unrounded coefficients, a wrong code range, a
flipped residual sign, and in the encoder's fixed fp32 order a reversed
summation order (step 1 or 2) and a wider (fp64) accumulator (step 1 or 2).

A separate multiply and add in place of the fused multiply-add is not a
mistake these pins could catch: every product in the encoder is of two fp16
values, which binary32 holds exactly, so both forms round once and give the
same bits (test_oracle_encoder_order.py proves the exactness)."""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_append as TA
from tests import test_oracle_decode as TD
from tests import test_oracle_encoder_order as TO
from tests import test_oracle_dense as TN
from tests import test_oracle_coef8 as TC

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

DECODE_PINS = [
    lambda: TD.test_identity_basis_equals_sdpa(1),
    TD.test_random_basis_equals_sdpa_on_materialised_cache,
    TD.test_full_rank_zero_residual_is_attention_on_BC,
    TD.test_single_token_returns_its_value,
    TD.test_two_tokens_logistic_weights,
    TD.test_zero_query_gives_mean_value,
    TD.test_constant_values_weights_sum_to_one,
    TD.test_planted_needle_is_returned,
]
APPEND_PINS = [
    lambda: TA.test_identity_basis_by_hand(4, 7, 0),
    lambda: TA.test_identity_basis_by_hand(8, 127, 1),
    TA.test_signed_permutation_basis_projects_exactly,
    TA.test_residual_matches_projection_residual_in_fp64,
    lambda: TA.test_kept_channels_are_best_subset_by_brute_force(0),
    lambda: TA.test_quantisation_error_bound(7),
    TA.test_ties_prefer_smaller_channel_and_zero_residual,
    TA.test_codes_round_half_to_even,
    lambda: TO.test_encoder_steps_match_exact_fma_chain(1, 8),
    lambda: TO.test_encoder_steps_match_exact_fma_chain(2, 64),
]

DENSE_PINS = [
    TN.test_materialize_matches_numpy_einsum,
    TN.test_materialize_identity_basis_is_exact,
    lambda: TN.test_dense_decode_equals_sdpa(0),
    TN.test_dense_decode_closed_forms,
]

COEF8_PINS = [
    TC.test_decode_with_8bit_coefficients_equals_sdpa_on_materialised_cache,
    TC.test_identity_basis_encoding_by_hand,
    lambda: TC.test_step2_against_exact_chain_with_dequantised_coefficients(16),
    TC.test_coefficient_quantisation_bound,
    TC.test_coefficient_codes_round_half_to_even,
]

_STEP1 = ("        float acc = 0.0f;                                         /* step 1 */\n"
          "        for (int j = 0; j < d; ++j)\n"
          "            acc = fmaf(h2f(basis[(int64_t)i * d + j]), h2f(x[j]), acc);\n")
_STEP2 = ("        float acc = 0.0f;                                         /* step 2 */\n"
          "        for (int i = 0; i < r; ++i)\n"
          "            acc = fmaf(h2f(basis[(int64_t)i * d + j]), c[i], acc);\n")

MUTANTS = {
    "drop_residual": ("x[idx[u]] += g * (double)val[u];", "(void)g;", DECODE_PINS),
    "residual_sign": ("x[idx[u]] += g * (double)val[u];", "x[idx[u]] -= g * (double)val[u];", DECODE_PINS),
    "kv_basis_swap": ("reconstruct(sh, bV, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, x);",
                      "reconstruct(sh, bK, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, x);",
                      DECODE_PINS),
    "head_map": ("q[((int64_t)b * Hq + h * gq + g) * d + j]", "q[((int64_t)b * Hq + g * Hkv + h) * d + j]",
                 DECODE_PINS),
    "no_softmax_scale": ("z[g * n + t] = alpha * acc;", "z[g * n + t] = acc;", DECODE_PINS),
    "rank_off_by_one": ("int r = sh->tier_rank[tier];", "int r = sh->tier_rank[tier] - 1;", DECODE_PINS),
    "basis_transposed": ("x[j] += c * bi[j];", "x[j] += c * basis[(int64_t)j * sh->r_max + i];", DECODE_PINS),
    "no_normalisation": ("o[g * d + j] /= den[g];", "o[g * d + j] /= 1.0;", DECODE_PINS),
    "exp2_weights": ("double w = exp(z[g * n + t] - mx[g]);", "double w = exp2(z[g * n + t] - mx[g]);",
                     DECODE_PINS),
    "tie_to_larger": ("fabsf(e[j]) > fabsf(e[best])", "fabsf(e[j]) >= fabsf(e[best])", APPEND_PINS),
    "round_half_away": ("v = rintf(e[j] / sf);", "v = roundf(e[j] / sf);", APPEND_PINS),
    "unrounded_coef": ("c[i] = h2f(c16[i]);", "c[i] = acc1[i];", APPEND_PINS),
    "wrong_code_range": ("amax / (float)qmax", "amax / (float)(qmax + 1)", APPEND_PINS),
    "residual_flipped": ("e[j] = h2f(x[j]) - acc;", "e[j] = acc - h2f(x[j]);", APPEND_PINS),
    "materialize_v_with_k_basis": ("reconstruct(sh, bV, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, xv);",
                                   "reconstruct(sh, bK, coefV, cscaleV, tt, idxV + tt * S, valV + tt * S, scaleV[tt], k, xv);",
                                   DENSE_PINS),
    "materialize_ragged_ignored": ("            if (t >= n_tokens[b]) {", "            if (t >= NM) {", DENSE_PINS),
    "dense_no_scale": ("            z[t] = alpha * acc;", "            z[t] = acc;", DENSE_PINS),
    "dense_head_map": ("int b = p / Hq, g = p % Hq, h = g / gq;", "int b = p / Hq, g = p % Hq, h = g % Hkv;",
                       DENSE_PINS),
    "dense_no_normalisation": ("            o[j] /= den;\n        free(z);", "            o[j] /= 1.0;\n        free(z);",
                               DENSE_PINS),
    "coef8_scale_range": ("*cs16 = oracle_float_to_half(amax / 127.0f);", "*cs16 = oracle_float_to_half(amax / 128.0f);",
                          COEF8_PINS),
    "coef8_residual_unquantised": ("            c[i] = q * sf;", "            c[i] = acc1[i];", COEF8_PINS),
    "coef8_round_away": ("                q = rintf(acc1[i] / sf);", "                q = roundf(acc1[i] / sf);",
                         COEF8_PINS),
    "coef8_scale_ignored": ("return oracle_half_to_double(cscale[tt]) * (double)((const int8_t *)coef)[tt * sh->r_max + i];",
                            "return (double)((const int8_t *)coef)[tt * sh->r_max + i];", COEF8_PINS),
    "step1_descending": (_STEP1, _STEP1.replace("for (int j = 0; j < d; ++j)", "for (int j = d - 1; j >= 0; --j)"),
                         APPEND_PINS),
    "step2_descending": (_STEP2, _STEP2.replace("for (int i = 0; i < r; ++i)", "for (int i = r - 1; i >= 0; --i)"),
                         APPEND_PINS),
    "step1_fp64_accumulate": (_STEP1, "        double acc64 = 0.0;\n"
                                      "        for (int j = 0; j < d; ++j)\n"
                                      "            acc64 = fma(h2f(basis[(int64_t)i * d + j]), h2f(x[j]), acc64);\n"
                                      "        float acc = (float)acc64;\n", APPEND_PINS),
    "step2_fp64_accumulate": (_STEP2, "        double acc64 = 0.0;\n"
                                      "        for (int i = 0; i < r; ++i)\n"
                                      "            acc64 = fma(h2f(basis[(int64_t)i * d + j]), c[i], acc64);\n"
                                      "        float acc = (float)acc64;\n", APPEND_PINS),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes_all_pins(workdir):
    so = os.path.join(workdir, "clean.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-ffp-contract=off", SRC, "-o", so,
                    "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle._load(so)
    try:
        for pin in DECODE_PINS + APPEND_PINS:
            pin()
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, workdir):
    old, new, pins = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(workdir, f"{name}.c")
    open(path, "w").write(src.replace(old, new))
    so = os.path.join(workdir, f"{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-ffp-contract=off", path, "-o", so,
                    "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle._load(so)
    caught = []
    try:
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught mutant {name}"
