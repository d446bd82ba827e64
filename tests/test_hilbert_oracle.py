"""The Hilbert token-order oracle against its pins, and planted mistakes against the pins."""
import os
import types

import pytest

import oracle.hilbert as hilbert
from tests import hilbert_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "hilbert.py")

MUTATIONS = {
    "reflect_and_swap_exchanged": ("            if x[i] & q:\n", "            if not x[i] & q:\n"),
    "gray_across_axes_skipped": ("        x[i] ^= x[i - 1]\n", "        pass\n"),
    "level_flip_skipped": ("    for i in range(n):\n        x[i] ^= flip\n", ""),
    "interleave_axes_reversed": ("h = (h << 1) | ((x[i] >> b) & 1)", "h = (h << 1) | ((x[n - 1 - i] >> b) & 1)"),
    "levels_interleaved_low_first": ("for b in range(bits - 1, -1, -1):", "for b in range(bits):"),
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
