"""Pins of the discarded-mass oracle (oracle/mass_oracle.py) against facts
that do not come from it: scipy's softmax, hand-derived values, the exact
identities of a truncated distribution and the EntmaxKV page's section-3
bound, and the alpha -> 1 limit."""
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import entmax_oracle as O
from oracle import mass_oracle as M


@pytest.mark.parametrize("seed", range(5))
def test_softmax_matches_scipy(seed):
    rng = np.random.default_rng(seed)
    for scale in (0.1, 3.0, 300.0):
        z = rng.normal(0.0, scale, 257)
        np.testing.assert_allclose(M.softmax(z), sp_softmax(z), rtol=1e-12, atol=1e-300)
    # large offsets: shift invariance, no overflow
    z = rng.normal(0.0, 1.0, 40) + 1000.0
    np.testing.assert_allclose(M.softmax(z), sp_softmax(z - 1000.0), rtol=1e-12)


def test_hand_example_alpha2():
    """z = (1, 0): sparsemax gives p = (1, 0) (the second token sits on the
    threshold), softmax gives (e/(1+e), 1/(1+e)). Keeping the first token
    drops no entmax mass but 1/(1+e) of softmax mass; the entmax output is
    exact, the softmax one is off by 1/(1+e) of (v1 - v2)."""
    z = np.array([1.0, 0.0])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    keep = np.array([True, False])
    r = M.mass_comparison(z, V, keep, 2.0)
    assert r["delta_entmax"] == 0.0
    assert r["delta_softmax"] == pytest.approx(1.0 / (1.0 + math.e), rel=1e-14)
    assert r["err_entmax"] == 0.0
    # full softmax output (e, 1)/(1+e); kept output (1, 0)
    assert r["err_softmax"] == pytest.approx(math.sqrt(2.0) / (1.0 + math.e), rel=1e-14)
    assert r["support"] == 1 and r["support_kept"] == 1


def test_uniform_scores_half_kept():
    """Uniform scores: both distributions are uniform, so keeping half the
    tokens drops half the mass under either."""
    n = 64
    z = np.full(n, 0.3)
    V = np.random.default_rng(1).normal(size=(n, 8))
    keep = np.arange(n) < n // 2
    for alpha in (1.25, 1.5, 2.0):
        r = M.mass_comparison(z, V, keep, alpha)
        assert r["delta_entmax"] == pytest.approx(0.5, rel=1e-12)
        assert r["delta_softmax"] == pytest.approx(0.5, rel=1e-12)
        np.testing.assert_allclose(M.entmax_kept_output(z, V, keep, alpha),
                                   V[:n // 2].mean(axis=0), rtol=1e-12)
        np.testing.assert_allclose(M.softmax_kept_output(z, V, keep), V[:n // 2].mean(axis=0),
                                   rtol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_l1_identity_and_section3_bound(alpha):
    """For both truncations ||p - p~||_1 = 2 delta exactly (re-solved entmax
    only grows on the kept set; renormalised softmax scales it by
    1/(1 - delta)), hence ||o - o~|| <= 2 B delta with B the largest value
    norm (the page's section-3 bound)."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        n = int(rng.integers(5, 200))
        z = rng.normal(0.0, 2.0, n)
        V = rng.normal(size=(n, 16))
        keep = rng.random(n) < 0.5
        keep[int(np.argmax(z))] = True
        r = M.mass_comparison(z, V, keep, alpha)
        p_e, _ = O.entmax(z, alpha)
        pk_e = np.zeros(n)
        pk_e[keep] = O.entmax(z[keep], alpha)[0]
        assert abs(np.abs(p_e - pk_e).sum() - 2 * r["delta_entmax"]) <= 1e-12
        p_s = M.softmax(z)
        pk_s = np.zeros(n)
        pk_s[keep] = M.softmax(z[keep])
        assert abs(np.abs(p_s - pk_s).sum() - 2 * r["delta_softmax"]) <= 1e-12
        assert r["err_entmax"] <= r["bound_entmax"] + 1e-12
        assert r["err_softmax"] <= r["bound_softmax"] + 1e-12
        # softmax drops mass whenever a token is dropped
        assert r["delta_softmax"] > 0.0


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_support_kept_means_no_entmax_error(alpha):
    rng = np.random.default_rng(3)
    n = 300
    z = rng.normal(0.0, 2.0, n)
    V = rng.normal(size=(n, 8))
    p, _ = O.entmax(z, alpha)
    keep = p > 0
    keep[rng.choice(n, 40, replace=False)] = True
    r = M.mass_comparison(z, V, keep, alpha)
    assert r["delta_entmax"] == 0.0 and r["support_kept"] == r["support"]
    assert r["err_entmax"] <= 1e-12 * np.linalg.norm(p @ V)
    assert r["delta_softmax"] > 0.0 and r["err_softmax"] > 1e-6


def test_entmax_mass_tends_to_softmax_mass():
    """alpha -> 1: the entmax distribution tends to softmax of the same
    scores (reading M1), so the dropped masses meet."""
    rng = np.random.default_rng(9)
    z = rng.normal(0.0, 1.0, 50)
    V = rng.normal(size=(50, 4))
    keep = np.arange(50) < 30
    ds = M.mass_comparison(z, V, keep, 2.0)["delta_softmax"]
    gaps = [abs(M.mass_comparison(z, V, keep, 1.0 + eps)["delta_entmax"] - ds)
            for eps in (1e-2, 1e-3, 1e-4)]
    assert gaps[0] > gaps[1] > gaps[2] and gaps[2] < 1e-3
