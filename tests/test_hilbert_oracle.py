"""The Hilbert token-order oracle against its pins, and planted mistakes against the pins."""
import os
import types

import pytest

import oracle.hilbert as hilbert
from tests import hilbert_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "hilbert.py")

MUTATIONS = {
    "gray_code_not_reflected": ("g = j ^ (j >> 1)", "g = j"),
    "axis0_least_significant": ("(g >> (n - 1 - a)) & 1", "(g >> a) & 1"),
    "first_quarter_not_mirrored": ("((1, 0), (0, 0)),  # (0,0)", "((0, 1), (0, 0)),  # (0,0)"),
    "last_quarter_not_flipped": ("((1, 0), (1, 1)),  # (1,0)", "((1, 0), (0, 0)),  # (1,0)"),
    "3d_first_piece_unrotated": ("((2, 0, 1), (0, 0, 0)),  # (0,0,0)", "((0, 1, 2), (0, 0, 0)),  # (0,0,0)"),
    "3d_fourth_piece_unflipped": ("((2, 1, 0), (1, 0, 1)),  # (0,1,0)", "((2, 1, 0), (0, 0, 0)),  # (0,1,0)"),
    "3d_seventh_piece_wrong_axes": ("((1, 0, 2), (1, 1, 0)),  # (1,0,1)", "((0, 1, 2), (1, 1, 0)),  # (1,0,1)"),
    "child_transform_skipped": ("hilbert_index(back, bits - 1)", "hilbert_index(y, bits - 1)"),
    "flip_over_the_whole_side": ("s - 1 - y[perm[a]] if flip[a]", "2 * s - 1 - y[perm[a]] if flip[a]"),
    "piece_weight_wrong": ("return j * s ** n +", "return j * s +"),
    "enclosing_cube_too_small": ("while any(s > (1 << k) for s in dims):", "while any(s > (2 << k) for s in dims):"),
    "not_sorted": ('order = np.argsort(keys, kind="stable")', "order = np.arange(len(keys))"),
    "text_moved_last": ("np.concatenate([np.arange(n_text), n_text + order])",
                        "np.concatenate([n_text + order, np.arange(n_text)])"),
    "inverse_is_gather": ("    out[..., perm, :] = x\n", "    out[...] = x[..., perm, :]\n"),
}


def test_oracle_passes_its_pins():
    assert hilbert_pins.failing(hilbert) == []


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutant_is_caught(name):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"anchor of {name} not found once"
    mod = types.ModuleType(f"hilbert_mutant_{name}")
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    assert hilbert_pins.failing(mod), f"no pin catches {name}"
