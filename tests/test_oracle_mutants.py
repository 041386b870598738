"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case below edits one line of a copy of ``oracle/diffattn_oracle.c`` into a
plausible slip (a wrong scale, sign, index, mask or normalisation), builds the
copy with gcc in a temporary directory, and runs the checks of
``test_oracle_pins.py`` against it.  At least one check must fail for every
mutant; the unmodified source must pass them all (``test_oracle_pins.py``).
"""
import os

import pytest

import oracle
from tests.test_oracle_pins import CHECKS

SRC = os.path.join(os.path.dirname(oracle.__file__), "diffattn_oracle.c")

MUTANTS = {
    "scale_by_sqrt_dv": ("1.0 / sqrt((double)d)", "1.0 / sqrt((double)dv)"),
    "no_score_scale": ("1.0 / sqrt((double)d)", "1.0"),
    "plus_lambda": ("a1[j] = a1[j] - lam * a2[j];", "a1[j] = a1[j] + lam * a2[j];"),
    "lambda_init_in_subtraction": ("a1[j] = a1[j] - lam * a2[j];",
                                   "a1[j] = a1[j] - lambda_init * a2[j];"),
    "maps_swapped_in_subtraction": ("a1[j] = a1[j] - lam * a2[j];",
                                    "a1[j] = a2[j] - lam * a1[j];"),
    "mask_one_too_wide": ("causal ? i + 1 : n_k", "causal ? (i + 2 < n_k ? i + 2 : n_k) : n_k"),
    "mask_strict": ("causal ? i + 1 : n_k", "causal ? (i > 0 ? i : 1) : n_k"),
    "map2_uses_k1": ("a2[j] = dot(q2i, k2 + j * d, d)", "a2[j] = dot(q2i, k1 + j * d, d)"),
    "map2_uses_q1": ("a2[j] = dot(q2i, k2 + j * d, d)", "a2[j] = dot(q1i, k2 + j * d, d)"),
    "value_transposed": ("D[c] += wj * vj[c];", "D[c] += wj * v[(int64_t)c * n_k + j]; (void)vj;"),
    "softmax_not_normalised": ("for (int64_t j = 0; j < n; ++j) x[j] /= z;",
                               "for (int64_t j = 0; j < n; ++j) x[j] /= (z + 1.0);"),
    "unbiased_variance": ("var /= dv;", "var /= (dv - 1);"),
    "eps_outside_sqrt": ("1.0 / sqrt(var + eps)", "1.0 / (sqrt(var) + eps)"),
    "no_eps": ("1.0 / sqrt(var + eps)", "1.0 / sqrt(var + 0.0 * eps)"),
    "no_output_scale": ("o[c] = (1.0 - lambda_init) * (D[c] - mu) * inv_std;",
                        "o[c] = (D[c] - mu) * inv_std;"),
    "lambda_init_as_scale": ("o[c] = (1.0 - lambda_init) * (D[c] - mu) * inv_std;",
                             "o[c] = lambda_init * (D[c] - mu) * inv_std;"),
    "no_mean_subtraction": ("o[c] = (1.0 - lambda_init) * (D[c] - mu) * inv_std;",
                            "o[c] = (1.0 - lambda_init) * D[c] * inv_std;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(path), lib=str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for check in CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name!r}"
