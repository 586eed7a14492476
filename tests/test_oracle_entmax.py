"""Pins of the oracle's alpha-entmax threshold and probabilities against
things other than itself: the variational definition solved by a generic
optimiser, the simplex projection (alpha = 2), softmax (alpha -> 1),
subset enumeration, hand-derived closed forms and invariants."""
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import minimize
from scipy.special import softmax

from oracle import entmax_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "entmax_worked_examples.json")


def tsallis_objective(p, z, alpha):
    """p.z + H_alpha(p), H_alpha(p) = sum (p - p^alpha) / (alpha (alpha-1))."""
    p = np.clip(p, 0.0, None)
    return float(p @ z + ((p - p ** alpha).sum()) / (alpha * (alpha - 1.0)))


def maximise_on_simplex(f, n, x0=None):
    x0 = np.full(n, 1.0 / n) if x0 is None else x0
    res = minimize(lambda p: -f(p), x0, method="SLSQP",
                   bounds=[(0.0, 1.0)] * n,
                   constraints=[{"type": "eq", "fun": lambda p: p.sum() - 1.0}],
                   options={"ftol": 1e-15, "maxiter": 2000})
    return res.x


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
@pytest.mark.parametrize("seed", range(6))
def test_entmax_maximises_tsallis_objective(alpha, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(3, 9))
    z = rng.normal(size=n) * 2.0
    p, _ = O.entmax(z, alpha)
    f = lambda x: tsallis_objective(x, z, alpha)
    p_opt = maximise_on_simplex(f, n)
    # The oracle's p is at least as good as the optimiser's point and close to it.
    assert f(p) >= f(p_opt) - 1e-10
    assert np.abs(p - p_opt).max() < 2e-4


@pytest.mark.parametrize("seed", range(8))
def test_sparsemax_is_euclidean_projection(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 12))
    z = rng.normal(size=n)
    p, tau = O.entmax(z, 2.0)
    proj = maximise_on_simplex(lambda x: -float(((x - z) ** 2).sum()), n)
    assert np.abs(p - proj).max() < 1e-5
    # With alpha = 2 the threshold is the projection's shift: p = [z - tau]_+.
    np.testing.assert_allclose(p, np.maximum(z - tau, 0.0), atol=1e-15)


def test_alpha_to_one_approaches_softmax():
    rng = np.random.default_rng(7)
    z = rng.normal(size=40) * 1.5
    ref = softmax(z)
    dists = []
    for eps in (1e-1, 1e-2, 1e-3, 1e-4):
        p, _ = O.entmax(z, 1.0 + eps)
        dists.append(np.abs(p - ref).sum())
    assert all(d2 < d1 for d1, d2 in zip(dists, dists[1:]))
    assert dists[-1] < 1e-3
    # roughly linear in eps
    assert dists[-1] / 1e-4 < 5.0 * dists[-2] / 1e-3 + 1e-9


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0, 1.1])
@pytest.mark.parametrize("seed", range(10))
def test_three_threshold_methods_agree(alpha, seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(1, 11))
    a = rng.normal(size=n) * rng.choice([0.2, 1.0, 3.0])
    t_sort = O.entmax_threshold(a, alpha)
    t_bis = O.entmax_threshold_bisect(a, alpha)
    t_brute, S = O.entmax_threshold_bruteforce(a, alpha)
    tol = 1e-10 * max(1.0, abs(t_sort))
    assert abs(t_sort - t_bis) <= tol
    assert abs(t_sort - t_brute) <= 1e-9 * max(1.0, abs(t_sort))
    p = O.entmax_probs(a, t_sort, alpha)
    assert set(np.nonzero(p > 0)[0].tolist()) == set(S)


def test_worked_examples_from_definition():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p, tau = O.entmax(np.array(c["z"], dtype=float), c["alpha"])
        np.testing.assert_allclose(tau, c["tau"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(p, c["p"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("n", [1, 2, 7, 100])
def test_uniform_scores(alpha, n):
    z = np.full(n, 0.37)
    p, tau = O.entmax(z, alpha)
    np.testing.assert_allclose(p, 1.0 / n, rtol=1e-12)
    np.testing.assert_allclose(tau, (alpha - 1) * 0.37 - n ** (-(alpha - 1)), atol=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 1.7])
@pytest.mark.parametrize("seed", range(5))
def test_invariants(alpha, seed):
    rng = np.random.default_rng(seed)
    n = 500
    z = rng.normal(size=n) * 4.0
    p, tau = O.entmax(z, alpha)
    a = (alpha - 1) * z
    assert (p >= 0).all()
    assert abs(p.sum() - 1.0) < 1e-12
    assert (p > 0).sum() >= 1
    # exact zeros outside the window, bracket on tau
    assert (p[a <= a.max() - 1.0] == 0).all()
    assert a.max() - 1.0 <= tau <= a.max() - n ** (-(alpha - 1)) + 1e-15
    # shift: same p, tau moves by (alpha-1) c
    c = 3.25
    p2, tau2 = O.entmax(z + c, alpha)
    np.testing.assert_allclose(p2, p, atol=1e-12)
    np.testing.assert_allclose(tau2, tau + (alpha - 1) * c, atol=1e-12)
    # permutation equivariance
    perm = rng.permutation(n)
    p3, _ = O.entmax(z[perm], alpha)
    np.testing.assert_allclose(p3, p[perm], atol=1e-14)
    # bisection over all scores lands on the same threshold
    assert abs(O.entmax_threshold_bisect(a, alpha) - tau) < 1e-11 * max(1, abs(tau))


def test_boundary_token_gets_zero():
    # alpha = 2, z = (1, 0): tau = 0 exactly and the second token sits on it.
    p, tau = O.entmax(np.array([1.0, 0.0]), 2.0)
    assert tau == 0.0 and p[1] == 0.0 and p[0] == 1.0


def test_sorted_search_uses_whole_window():
    # Many nearly tied top scores: the support must take all of them.
    z = np.concatenate([np.full(50, 10.0) + np.linspace(0, 1e-3, 50), np.zeros(10)])
    for alpha in (1.25, 1.5, 2.0):
        p, _ = O.entmax(z, alpha)
        assert (p[:50] > 0).all() and (p[50:] == 0).all()
