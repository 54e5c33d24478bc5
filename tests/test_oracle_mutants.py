"""The pins are sharp enough: planted mistakes in the oracle fail them.

Each case copies oracle/mha_oracle.c, plants one plausible mistake by text
substitution (a dropped term, a wrong sign or index, a transposed operand),
compiles the copy with gcc into a temporary directory, points the oracle
wrapper at it, and checks that at least one pin test now fails.  Everything
happens on the CPU; the real oracle is untouched.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_ex_pins as ex
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mha_oracle.c")

MUTANTS = {
    "scale_dropped": ("s_row[j] = scale * dot - rv->slope * dist;",
                      "s_row[j] = dot - rv->slope * dist;"),
    "causal_reversed": ("(rv->mode == 0 || j <= rv->pos)", "(rv->mode == 0 || j >= rv->pos)"),
    "padding_off_by_one": ("return j < rv->L &&", "return j <= rv->L &&"),
    "not_normalised": ("a_row[j] /= Z;", "a_row[j] /= 1.0;"),
    "value_row_reversed": ("const double *v = Vh + j * dv;",
                           "const double *v = Vh + (m - 1 - j) * dv;"),
    "key_uses_query_index": ("const double *k = Kh + j * dk;",
                             "const double *k = Kh + (rv->pos >= 0 && rv->pos < m ? rv->pos : j) * dk;"),
    "feature_sum_truncated": ("for (int64_t c = 0; c < dk; ++c) dot += q[c] * k[c];",
                              "for (int64_t c = 0; c + 1 < dk; ++c) dot += q[c] * k[c];"),
    "max_not_subtracted": ("exp(s_row[j] - M)", "exp(s_row[j])"),
    # the extended operation
    "alibi_sign": ("scale * dot - rv->slope * dist", "scale * dot + rv->slope * dist"),
    "alibi_distance_signed": ("if (dist < 0) dist = -dist;", "if (dist < 0) dist = dist;"),
    "kv_head_interleaved": ("t / group;", "t % Hkv;"),
    "bottom_right_offset_sign": ("i + rv.L - n", "i + n - rv.L"),
    "lse_log_dropped": ("*lse = M + log(Z);", "*lse = M + Z;"),
    "lse_max_dropped": ("*lse = M + log(Z);", "*lse = log(Z);"),
}

PIN_TESTS = [
    lambda: pins.test_worked_example_4token_printed_values(),
    lambda: pins.test_worked_example_4token_closed_form(),
    lambda: pins.test_causal_3x3_example(),
    lambda: pins.test_saturation_example(),
    lambda: pins.test_large_scores_stay_finite(),
    lambda: pins.test_rows_sum_to_one_and_masked_are_zero(True),
    lambda: pins.test_self_attention_permutation_equivariant(),
    lambda: pins.test_causal_row0_is_v0(),
    lambda: pins.test_zero_query_gives_mean_of_valid_values(True),
    lambda: pins.test_brute_force_tiny(False),
    lambda: pins.test_brute_force_tiny(True),
    lambda: pins.test_matches_torch_sdpa_float64(False, 11, 30),
    lambda: pins.test_padding_content_has_no_effect(False),
    lambda: ex.test_gqa_matches_torch_head_mapping(2),
    lambda: ex.test_bottom_right_matches_torch_lower_right_bias(3, 9),
    lambda: ex.test_one_decode_query_sees_the_whole_prefix(),
    lambda: ex.test_alibi_matches_sdpa_with_float_bias(False),
    lambda: ex.test_alibi_zero_query_closed_form(0.3),
    lambda: ex.test_lse_worked_example_printed_sum(),
    lambda: ex.test_lse_matches_scipy_logsumexp("bottom_right"),
]


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) >= 1, "mutation site for %s not found" % name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(text.replace(old, new), encoding="utf-8")
    lib = tmp_path / ("mutant_%s.so" % name)
    cmd = [c for c in oracle.GCC_CMD if c not in (oracle._SRC, oracle._LIB)]
    cmd = [c for c in cmd if c not in ("-o", "-lm")] + [str(src), "-o", str(lib), "-lm"]
    subprocess.run(cmd, check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, monkeypatch, name):
    path = _build_mutant(tmp_path, name)
    # Load the mutant through the wrapper's own ctypes set-up.
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB", path)
    monkeypatch.setattr(oracle, "build", lambda force=False: path)
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
        except (ValueError, FloatingPointError):
            caught += 1
    assert caught > 0, "no pin caught the planted mistake %r" % name


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    lib = tmp_path / "copy.so"
    cmd = list(oracle.GCC_CMD)
    cmd[cmd.index(oracle._LIB)] = str(lib)
    subprocess.run(cmd, check=True)
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB", str(lib))
    monkeypatch.setattr(oracle, "build", lambda force=False: str(lib))
    for t in PIN_TESTS:
        t()
    ctypes.CDLL(str(lib))
