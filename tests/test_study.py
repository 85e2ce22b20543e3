"""Host checks of the error-propagation study's measurement helpers: the rank
correlation against scipy's (ties included) and closed forms, the half-life
of a constant retention, and the study's tables."""
import math

import numpy as np
import pytest
from scipy import stats

from quantized_delta_rule_decode_amd import study, synth


def test_spearman_matches_scipy_with_ties():
    g = np.random.default_rng(3)
    for n in (5, 17, 300):
        x = g.integers(0, 7, size=n).astype(float)       # many ties
        y = x * 0.5 + g.standard_normal(n)
        assert study.spearman(x, y) == pytest.approx(stats.spearmanr(x, y).statistic, abs=1e-12)
        x = g.standard_normal(n)
        y = g.standard_normal(n)
        assert study.spearman(x, y) == pytest.approx(stats.spearmanr(x, y).statistic, abs=1e-12)


def test_spearman_closed_forms():
    x = np.arange(10.0)
    assert study.spearman(x, x ** 3) == pytest.approx(1.0)      # any increasing map
    assert study.spearman(x, -np.exp(x)) == pytest.approx(-1.0)
    # rho = 1 - 6 sum d^2 / (n (n^2 - 1)) without ties: swap two neighbours
    y = x.copy()
    y[[3, 4]] = y[[4, 3]]
    n = x.size
    assert study.spearman(x, y) == pytest.approx(1 - 6 * 2 / (n * (n * n - 1)))
    assert study.ranks([3.0, 1.0, 3.0, 2.0]).tolist() == [3.5, 1.0, 3.5, 2.0]


def test_halflife_of_retention():
    hl = np.array([1.0, 2.5, 100.0, 4096.0])
    alpha = 2.0 ** (-1.0 / hl)
    assert np.allclose(study.halflife(alpha), hl, rtol=1e-12)
    assert np.allclose(alpha ** study.halflife(alpha), 0.5)


def test_study_tables():
    sc = study.StudyConfig(H=40, B=2, T=3)
    t = study.study_tables(sc)
    assert (t["kinds"] == synth.INT6).all() and t["kinds"].size == 40
    cfg = sc.synth_config()
    assert cfg.scale_mode == synth.SCALE_ROW_ABSMAX and cfg.gate_mode == "per_head" and cfg.warmup == 0
    # the gate the steps use is the float32 retention of the listed half-life
    # (float32 rounding of alpha near 1 moves the half-life by up to ~1e-4)
    assert np.allclose(study.halflife(t["alpha_head"]), t["halflife"], rtol=1e-3)
    assert 1.0 <= t["halflife"].min() and t["halflife"].max() <= 4096.0
    q, k, v, beta, gate = synth.step_inputs(cfg, t, 0)
    assert gate.shape == (2, 40) and np.array_equal(gate[1], t["alpha_head"])
