"""Pins of the Gaussian-aware selection oracle against facts that do not come
from the oracle itself: numerical integration, textbook values, the exact
entmax threshold it reduces to when every page is a single token, Monte
Carlo, and brute force over tiny cases."""
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import entmax_oracle as O
from oracle import gauss_oracle as GO

ALPHAS = (2.0, 1.5, 4.0 / 3.0, 1.25)


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("c", [-6.0, -2.0, -0.5, 0.0, 0.7, 3.0, 7.0])
def test_partial_moment_matches_quadrature(m, c):
    """E[(Y - c)_+^m] against adaptive quadrature of (y - c)^m phi(y)."""
    f = lambda y: (y - c) ** m * math.exp(-0.5 * y * y) / math.sqrt(2 * math.pi)
    ref, err = integrate.quad(f, c, np.inf, epsabs=1e-15, epsrel=1e-12)
    got = float(GO.normal_partial_moment(c, m))
    assert abs(got - ref) <= 1e-10 * max(1.0, abs(ref)) + 1e-14, (got, ref, err)


def test_partial_moment_textbook_values():
    # E[Y_+] = 1/sqrt(2 pi); E[Y_+^2] = 1/2; E[Y_+^3] = 2/sqrt(2 pi); E[Y_+^4] = 3/2
    assert GO.normal_partial_moment(0.0, 1) == pytest.approx(1 / math.sqrt(2 * math.pi), rel=1e-15)
    assert GO.normal_partial_moment(0.0, 2) == pytest.approx(0.5, rel=1e-15)
    assert GO.normal_partial_moment(0.0, 3) == pytest.approx(2 / math.sqrt(2 * math.pi), rel=1e-15)
    assert GO.normal_partial_moment(0.0, 4) == pytest.approx(1.5, rel=1e-15)
    # far left: (Y - c)_+ = Y - c almost surely, so the raw moments of Y + |c|
    c = -40.0
    assert GO.normal_partial_moment(c, 1) == pytest.approx(40.0, rel=1e-15)
    assert GO.normal_partial_moment(c, 2) == pytest.approx(1600.0 + 1.0, rel=1e-14)


@pytest.mark.parametrize("alpha", ALPHAS)
def test_threshold_reduces_to_exact_entmax_for_point_pages(alpha):
    """Pages of one token each with zero variance: the approximate equation is
    the exact alpha-entmax equation, so tau_hat is the entmax threshold."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 7, 50, 300):
        a = rng.normal(0.0, 1.5, n)
        tau_hat = GO.gauss_threshold(a, np.zeros(n), np.ones(n), alpha)
        # the exact threshold for the exponent m = 1/(alpha-1) the selection uses
        tau = O.entmax_threshold(a, 1.0 + 1.0 / GO.integer_m(alpha))
        assert abs(tau_hat - tau) <= 1e-12 * max(1.0, abs(tau)), (n, tau_hat, tau)


@pytest.mark.parametrize("alpha", (1.5, 1.25))
def test_threshold_with_repeated_point_pages(alpha):
    """A zero-variance page of n tokens counts like n copies of its score."""
    a = np.array([2.0, 1.7, 0.4, -1.0])
    n = np.array([3, 1, 5, 2])
    tau_hat = GO.gauss_threshold(a, np.zeros(4), n, alpha)
    tau = O.entmax_threshold(np.repeat(a, n), 1.0 + 1.0 / GO.integer_m(alpha))
    assert abs(tau_hat - tau) <= 1e-12 * max(1.0, abs(tau))


@pytest.mark.parametrize("alpha", ALPHAS)
def test_threshold_satisfies_equation_by_monte_carlo(alpha):
    """At tau_hat, a Monte Carlo estimate of sum_p n_p E[(A_p - t)_+^m] is 1
    within its sampling error (an independent evaluation of the expectation)."""
    rng = np.random.default_rng(5)
    m = GO.integer_m(alpha)
    P = 6
    mu = rng.normal(0.0, 0.6, P)
    s = rng.uniform(0.05, 0.5, P)
    n = rng.integers(4, 40, P)
    tau_hat = GO.gauss_threshold(mu, s, n, alpha)
    N = 400_000
    vals = []
    for p in range(P):
        draws = rng.normal(mu[p], s[p], N)
        vals.append(n[p] * np.maximum(draws - tau_hat, 0.0) ** m)
    per_draw = np.sum(vals, axis=0)
    est, se = per_draw.mean(), per_draw.std() / math.sqrt(N)
    assert abs(est - 1.0) <= 5 * se + 1e-12, (est, se)


@pytest.mark.parametrize("alpha", ALPHAS)
def test_expected_mass_is_decreasing_and_brackets(alpha):
    m = GO.integer_m(alpha)
    rng = np.random.default_rng(3)
    mu, s, n = rng.normal(0, 1, 20), rng.uniform(0, 0.8, 20), rng.integers(1, 33, 20)
    s[::5] = 0.0
    ts = np.linspace(mu.max() - 1.0, (mu + 40 * s).max(), 200)
    f = [GO.expected_mass(t, mu, s, n, m) for t in ts]
    assert f[0] >= 1.0 and f[-1] < 1e-12
    assert all(x >= 0.0 for x in f)
    assert all(x >= y - 1e-250 for x, y in zip(f, f[1:]))


def test_integer_m_rejects_other_alphas():
    for alpha in (1.1, 1.4, 3.0, 1.6):
        with pytest.raises(ValueError):
            GO.integer_m(alpha)
    assert [GO.integer_m(a) for a in ALPHAS] == [1, 2, 3, 4]


def test_estimated_max_single_token_and_monotone():
    """A page of one token is its own maximum (no spread); the estimate grows
    with the page's token count and is affine in (mu, s)."""
    est = GO.estimated_max([1.0, -2.0], [0.5, 3.0], [1, 1])
    assert est[0] == 1.0 and est[1] == -2.0
    ns = np.array([1, 2, 4, 16, 64, 1024])
    e = GO.estimated_max(np.zeros(len(ns)), np.ones(len(ns)), ns)
    assert np.all(np.diff(e) > 0)
    a = GO.estimated_max([0.3], [0.7], [64])[0]
    b = GO.estimated_max([0.0], [1.0], [64])[0]
    assert a == pytest.approx(0.3 + 0.7 * b, rel=1e-15)


def _expected_max_std_normal(n):
    """E[max of n iid N(0,1)] by quadrature of x n phi(x) Phi(x)^(n-1)."""
    from scipy import stats
    f = lambda x: x * n * stats.norm.pdf(x) * stats.norm.cdf(x) ** (n - 1)
    val, _ = integrate.quad(f, -12.0, 12.0, limit=400, points=[0.0, 2.0, 4.0])
    return val


def test_expected_max_quadrature_textbook():
    """The quadrature used below gives the textbook E[max of 2 N(0,1)] =
    1/sqrt(pi)."""
    assert _expected_max_std_normal(2) == pytest.approx(1.0 / math.sqrt(math.pi), rel=1e-9)


@pytest.mark.parametrize("n", [16, 32, 64])
def test_estimated_max_against_simulated_maximum(n):
    """Reading G4 takes a page's estimated maximum as the usual growth of the
    largest of n Gaussian draws. Checked against the maximum itself,
    simulated (seeded Monte Carlo, 100000 pages of n draws from N(mu, s^2)):
    the estimate lies above the simulated mean maximum (sqrt(2 ln n) bounds
    E[max] of n standard normals), by less than s times the classical
    second-order term (ln ln n + ln 4 pi) / (2 sqrt(2 ln n)) of the
    maximum's growth, and the simulated mean agrees with the quadrature of
    E[max]. A dropped factor, a wrong logarithm, s^2 for s or a sign error
    in mu each breaks one of these."""
    mu, s = 0.7, 0.3
    rng = np.random.default_rng(100 + n)
    N = 100_000
    mx = rng.normal(mu, s, (N, n)).max(axis=1)
    m_hat, se = float(mx.mean()), float(mx.std() / math.sqrt(N))
    assert abs(m_hat - (mu + s * _expected_max_std_normal(n))) <= 5 * se
    est = float(GO.estimated_max([mu], [s], [n])[0])
    r = math.sqrt(2.0 * math.log(n))
    second = (math.log(math.log(n)) + math.log(4.0 * math.pi)) / (2.0 * r)
    assert est > m_hat + 5 * se
    assert est - m_hat < s * second - 5 * se
    # and it is a high quantile of the simulated maximum, not its median
    frac_below = float((mx <= est).mean())
    assert 0.80 < frac_below < 0.95


def test_near_threshold_hand_cases():
    """Hand-computed near-threshold sets (reading G5's excusal band)."""
    # cut = tau_hat - delta = 1.5; band 1e-9 * max(1, |tau_hat|) = 2e-9
    est = [1.0, 2.0, 1.5 + 5e-10, 1.5 - 5e-10, 1.5 + 1e-8, 3.0]
    assert GO.gauss_near_threshold(est, 2.0, 0.5, 6) == {2, 3}
    # cap 2 binds (pages 1..5 pass): float32 keys 3, 2, 1.5, 1.5, 1.5; the
    # cap-th key is 2.0 and page 1 sits on it
    assert GO.gauss_near_threshold(est, 2.0, 0.5, 2) == {1, 2, 3}
    # cap boundary among float32 ties: 4 +- 1e-7 both round to 4.0
    est2 = [5.0, 4.0, 4.0 + 1e-7, 4.0 - 1e-7, 1.0]
    assert GO.gauss_near_threshold(est2, 0.0, 0.0, 2) == {1, 2, 3}
    # nothing near when every estimate is far from the cut and the cap does
    # not bind
    assert GO.gauss_near_threshold([0.0, 1.0, 2.0], 0.5, 0.0, 3) == set()
    # a wider band (relative to |tau_hat| = 10) takes in more pages
    est3 = [10.0 + 5e-9, 10.0 + 5e-8, 9.0]
    assert GO.gauss_near_threshold(est3, 10.0, 0.0, 3) == {0}
    assert GO.gauss_near_threshold(est3, 10.0, 0.0, 3, rel=1e-8) == {0, 1}


def test_selection_of_point_pages_is_the_support():
    """Single-token, zero-variance pages with Delta = 0: the selected pages are
    exactly those holding a support token (a_i > tau) of exact entmax."""
    rng = np.random.default_rng(8)
    for alpha in ALPHAS:
        a = rng.normal(0.0, 2.0, 200)
        tau_hat = GO.gauss_threshold(a, np.zeros(200), np.ones(200), alpha)
        est = GO.estimated_max(a, np.zeros(200), np.ones(200))
        sel = [j for j in GO.gauss_select_pages(est, tau_hat, 0.0, 200) if j >= 0]
        tau = O.entmax_threshold(a, 1.0 + 1.0 / GO.integer_m(alpha))
        support = [j for j in range(200) if a[j] > tau]
        assert sel == support


def test_selection_margin_cap_and_order():
    est = np.array([0.5, 2.0, 1.0, 2.0, -3.0, 1.5])
    # no margin: above 1.2
    assert GO.gauss_select_pages(est, 1.2, 0.0, 6) == [1, 3, 5, -1, -1, -1]
    # a larger margin keeps a superset
    assert GO.gauss_select_pages(est, 1.2, 0.8, 6) == [0, 1, 2, 3, 5, -1]
    # the cap keeps the largest estimates, ties to the lower page
    assert GO.gauss_select_pages(est, 1.2, 0.8, 3) == [1, 3, 5]
    assert GO.gauss_select_pages(est, 1.2, 0.8, 1) == [1]
    # brute force over every margin: monotone supersets
    prev = set()
    for d in np.linspace(0, 6, 25):
        cur = {j for j in GO.gauss_select_pages(est, 1.2, d, 6) if j >= 0}
        assert prev <= cur
        prev = cur
    assert prev == set(range(6))


def test_round_to_kv_bf16_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3, 1.0 + 2 ** -9])
    got = GO.round_to_kv(vals, "bf16")
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: to even (1); 1 + 3*2^-8 -> 1 + 2^-6
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2 ** -6
    assert got[3] == -2.5
    assert abs(got[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3
    assert got[5] == 1.0
    assert np.array_equal(GO.round_to_kv(vals, "f32"), vals.astype(np.float32).astype(np.float64))


def test_page_moments_closed_forms():
    """Identical rows: mean = the row, var = 0; two rows a, b: mean (a+b)/2,
    var ((a-b)/2)^2 (values exact in bf16)."""
    D = 8
    ps = 4
    k = np.zeros((2, 1, ps, D), dtype=np.float32)
    row = np.linspace(-1.5, 2.0, D).astype(np.float32)
    k[0, 0, :, :] = row
    k[1, 0, 0, :] = 1.0
    k[1, 0, 1, :] = 3.0
    bt = np.array([[0], [1]], dtype=np.int32)
    lens = np.array([4, 2], dtype=np.int32)
    mean, var = GO.page_moments(k, bt, lens, ps, "f32")
    assert np.array_equal(mean[0, 0], row.astype(np.float64)) and np.all(var[0, 0] == 0.0)
    assert np.all(mean[1, 0] == 2.0) and np.all(var[1, 0] == 1.0)


def test_page_score_stats_definition():
    q = np.array([1.0, -2.0, 0.5])
    mean = np.array([0.5, 0.25, -1.0])
    var = np.array([1.0, 0.5, 4.0])
    mu_a, s_a = GO.page_score_stats(q, mean, var, 1.5)
    assert mu_a == pytest.approx(0.5 * (0.5 - 0.5 - 0.5))
    assert s_a == pytest.approx(0.5 * math.sqrt(1.0 + 2.0 + 1.0))
