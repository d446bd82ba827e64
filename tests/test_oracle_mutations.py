"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Every mutant is built from the oracle's source text with one edit and loaded as
a separate module; the real oracle is never modified.
"""
import importlib.util
import os
import types

import pytest

from tests import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rettention.py")

MUTATIONS = {
    "residual_exponent_sign": ("r_c * np.exp(m_c - big)", "r_c * np.exp(big - m_c)"),
    "ratio_inverted": ("z_full_c / z_sparse_c", "z_sparse_c / z_full_c"),
    "residual_dropped": ("+ r_c * np.exp(m_c - big)[:, None]", ""),
    "residual_over_kept_keys": ("r = p[:, ~kept] @ V[~kept]", "r = p[:, kept] @ V[kept]"),
    "sparse_denominator_is_full": ("z_sparse = p[:, kept].sum(axis=1)", "z_sparse = p.sum(axis=1)"),
    "scale_uses_d_not_sqrt": ("alpha = dtype(1.0) / np.sqrt(dtype(d))", "alpha = dtype(1.0) / dtype(d)"),
    "short_block_divided_by_64": ("/ dtype(b - a) for a, b", "/ dtype(block) for a, b"),
    "tie_break_reversed": ("(-float(srow[j]), j)", "(-float(srow[j]), -j)"),
    "ascending_scores_kept": ("(-float(srow[j]), j)", "(float(srow[j]), j)"),
    "forced_not_counted": ("rest[: keep - len(fixed)]", "rest[:keep]"),
    "max_not_subtracted_in_sparse": ("p = np.exp(s - m[:, None])\n    z = p.sum(axis=1)",
                                     "p = np.exp(s)\n    z = p.sum(axis=1)"),
    "current_max_scale_dropped": ("n * np.exp(m - big)[:, None]", "n"),
    "kept_block_off_by_one": ("mask[j * block: min((j + 1) * block, N)] = True",
                              "mask[(j + 1) * block: min((j + 2) * block, N)] = True"),
    "r2_ratio_inverted": ("(z_sparse_c / z_full_c)[:, None] * o_sparse", "(z_full_c / z_sparse_c)[:, None] * o_sparse"),
    "r2_residual_over_sparse_denominator": ("+ r_c / z_full_c[:, None]", "+ r_c / z_sparse_c[:, None]"),
    "r2_sparse_output_unnormalised": ("o_sparse = (p @ V) / p.sum(axis=1)[:, None]", "o_sparse = p @ V"),
    "r2_residual_dropped": ("* o_sparse + r_c / z_full_c[:, None]", "* o_sparse"),
    # dense attention (the reference of the GPU identity tests)
    "dense_scale_uses_d_not_sqrt": ("alpha = dtype(1.0) / np.sqrt(dtype(d))\n    o = np.zeros(",
                                    "alpha = dtype(1.0) / dtype(d)\n    o = np.zeros("),
    "dense_max_over_wrong_axis": ("p = np.exp(s - s.max(axis=1, keepdims=True))",
                                  "p = np.exp(s - s.max(axis=0, keepdims=True))"),
    "dense_max_not_subtracted": ("p = np.exp(s - s.max(axis=1, keepdims=True))", "p = np.exp(s)"),
    "dense_normalised_by_max": ("(p @ V) / p.sum(axis=1, keepdims=True)", "(p @ V) / p.max(axis=1, keepdims=True)"),
    "dense_values_misaligned": ("K, V = k[b, h, :N], v[b, h, :N]", "K, V = k[b, h, :N], v[b, h, :N][::-1]"),
    "dense_keys_of_own_block_only": ("s = alpha * (q[b, h, a:e] @ K.T)", "s = alpha * (q[b, h, a:e] @ K[a:e].T)"),
}


def load_mutant(name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor for {name} not found"
    text = text.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(text, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_all_pins():
    spec = importlib.util.spec_from_file_location("oracle_copy", SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert pins.failing_pins(mod) == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutant_is_caught(name):
    assert pins.failing_pins(load_mutant(name)), f"no pin catches mutation {name}"
