"""CPU checks of the oracle against facts outside itself (no GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from sparse_attention_diffusion_amd import configs, synth
from tests import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name", list(pins.ALL_PINS))
def test_pin(name):
    fn, tol = pins.ALL_PINS[name]
    err = fn(oracle)
    assert err <= tol, (name, err)


@pytest.mark.parametrize("N,d,D,keep,forced", [
    (64, 8, 8, 1, ()),          # one block: everything kept
    (100, 8, 8, 1, ()),         # short last block
    (192, 64, 64, 2, (0,)),
    (130, 72, 80, 3, (2,)),     # padded head dim, scale from the true dim
    (256, 16, 16, 4, ()),       # keep all
    (256, 16, 16, 1, (3,)),     # only the forced block
])
def test_closed_form_tiny(N, d, D, keep, forced):
    err = pins.pin_closed_form(oracle, N=N, d=d, D=D, keep=keep, forced=forced, seed=N + d)
    assert err <= 1e-10, err


def test_closed_form_tiny_workload():
    """The 2-step tiny workload (16x16 grid, fp32, keep 2 of 4) end to end."""
    cfg = configs.CONFIGS["tiny"]
    (q0, k0, v0), (q1, k1, v1) = synth.steps(cfg, 2, seed=0)
    N, d = cfg["N"], cfg["d"]
    idx = oracle.select_blocks(q0, k0, N, d, cfg["keep"], configs.forced_blocks(cfg))
    st = oracle.calibrate(q0, k0, v0, idx, N, d)
    o = oracle.sparse_reshape(q1, k1, v1, idx, st, N, d)
    ref = oracle.closed_form_fp64(q1, k1, v1, q0, k0, v0, idx, N, d)
    assert pins.rel(o, ref) < 1e-10
    # float32 evaluation of the same formulation stays close to the float64 one
    st32 = oracle.calibrate(q0, k0, v0, idx, N, d, dtype=np.float32)
    o32 = oracle.sparse_reshape(q1, k1, v1, idx, st32, N, d, dtype=np.float32)
    assert pins.rel(o32, ref) < 1e-5


def test_select_matches_full_sort_per_row():
    rng = np.random.default_rng(0)
    for nb in (4, 16, 64, 278):
        s = rng.standard_normal((nb,)).astype(np.float32)
        keep = min(9, nb)
        forced = [0, 1, 2, 3][: min(4, keep - 1)]
        got = oracle.select_from_scores(s, keep, forced)
        order = sorted((j for j in range(nb) if j not in forced), key=lambda j: (-s[j], j))
        assert got == sorted(forced + order[: keep - len(forced)])


def test_select_negative_zero_ties():
    s = np.array([0.0, -0.0, 0.0, -1.0], dtype=np.float32)
    assert oracle.select_from_scores(s, 2, []) == [0, 1]


def test_page_figures():
    """Sparsity of the video workloads against the figures the project page prints."""
    figs = {f["name"]: f for f in json.load(open(os.path.join(HERE, "golden", "page_figures.json")))["figures"]}
    for name in ("cogvideox2b", "cogvideox5b"):
        cfg = configs.CONFIGS[name]
        N, d, keep = cfg["N"], cfg["d"], cfg["keep"]
        nb = configs.n_blocks(N)
        frac_blocks = keep / nb
        assert abs(frac_blocks - figs["kept_token_fraction"]["value"]) < 0.002
        # any valid list: forced text blocks + 5 others; take the worst case (full blocks)
        idx = np.tile(np.arange(keep, dtype=np.int32), (1, 1, nb, 1))
        dense = 4 * d * N * N
        assert 1 - oracle.kept_flops(idx, N, d) / dense > figs["skipped_attention_fraction"]["value"]
        assert configs.forced_blocks(cfg) == [0, 1, 2, 3]


def test_kept_flops_counts_partial_blocks():
    idx = np.array([[[[0, 1], [1, 2], [0, 2]]]], dtype=np.int32)  # N = 150: blocks 64, 64, 22
    assert oracle.kept_flops(idx, 150, 8) == 4 * 8 * (64 * 128 + 64 * 86 + 22 * 86)


def test_generator_deterministic_and_padded():
    cfg = dict(configs.CONFIGS["pixart512"], B=1, H=2)
    a = synth.steps(cfg, 2, seed=0)
    b = synth.steps(cfg, 2, seed=0)
    c = synth.steps(cfg, 1, seed=1)
    for (x, y) in zip(a[1], b[1]):
        assert bool((x.float() == y.float()).all())
    assert not bool((a[0][0].float() == c[0][0].float()).all())
    for t in a[0]:
        assert t.dtype.is_floating_point and t.shape == (1, 2, 1024, 80)
        assert float(t[..., 72:].abs().max()) == 0.0


def test_generator_statistics():
    """Field variance 4 * 1/2 plus noise variance 0.25; drift keeps it near constant."""
    cfg = dict(configs.CONFIGS["pixart1024"], B=1, H=2)
    it = synth.StepInputs(cfg, seed=0)
    q, _, _ = it.next()
    var0 = float(q[..., :72].var())
    assert 1.8 < var0 < 2.7
    for _ in range(3):
        q, _, _ = it.next()
    assert 1.5 < float(q[..., :72].var()) < 2.8


def test_generator_text_tokens():
    cfg = dict(configs.CONFIGS["cogvideox2b"], B=1, H=1)
    q, k, v = synth.StepInputs(cfg, seed=0).next()
    text = q[0, 0, :226, :64]
    assert abs(float(text.mean())) < 0.05 and 0.9 < float(text.std()) < 1.1
    assert synth.coords(cfg).shape == (13 * 30 * 45, 3)
