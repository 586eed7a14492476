"""Plain fp64 CPU oracle for the Gaussian-aware entmax page selection of the
EntmaxKV method.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The library (the HIP path) never
imports, links or runs it, and this module imports nothing from the library.

Source: "Riepilogo Tecnico: EntmaxKV - Decodifica Consapevole del Supporto
per l'Attention Entmax" (gist.science, paper 2605.21649), [EntmaxKV page]:
  - section 2.A, second bullet: each page also keeps the first and second
    moments (mean and variance) of its keys, so that the scores of a page's
    tokens can be treated as a Gaussian random variable;
  - section 2.B, policy 2: tau is estimated from those page-level Gaussians by
    solving an approximate normalisation equation, and the pages whose
    estimated maximum score exceeds the estimate (less a safety margin Delta)
    are selected, so the number of pages follows the query's scores.
The pages state neither the equation, nor the estimator of a page's maximum,
nor Delta. The readings taken here:
  G1  moments: per coordinate, the mean and the population variance (1/n) of
      the page's valid keys, computed in float64 and stored in the cache's
      dtype, rounded through float32 (float64 -> float32 -> bf16, each round
      to nearest even);
  G2  the scores z = q.k of a page's tokens ~ N(mu, s^2) with
      mu = sum_d q_d mean_d and s^2 = sum_d q_d^2 var_d (coordinates taken as
      independent); in the units of tau, a = (alpha-1) z ~ N(mu_a, s_a^2);
  G3  the approximate normalisation: sum_p n_p E[(A_p - t)_+^m] = 1, with
      n_p the page's valid tokens and m = 1/(alpha-1); tau_hat is its root.
      Closed forms exist for integer m, so alpha is limited to 2, 3/2, 4/3
      and 5/4 (m = 1..4);
  G4  a page's estimated maximum: mu_a + s_a sqrt(2 ln n_p) (the usual
      growth of the largest of n Gaussian draws; mu_a alone when n_p = 1);
  G5  selected: the pages with estimated maximum > tau_hat - Delta (Delta >= 0
      in the units of tau, a caller parameter); when more than `cap` pages
      qualify, the cap with the largest estimate rounded to float32, ties to
      the lower page index. Listed ascending, padded with -1.
Every function works in float64. Pins: tests/test_oracle_gauss.py.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc

from .entmax_oracle import kv_to_f64, num_pages, page_rows

# ---------------------------------------------------------------------------
# [EntmaxKV page] section 2.A, Gaussian statistics (readings G1)


def round_to_kv(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored value of a float64 statistic: float64 -> float32 (nearest even)
    and, for bf16 caches, float32 -> bf16 (nearest even); returned widened to
    float64."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if kv_dtype == "f32":
        return f32.astype(np.float64)
    if kv_dtype != "bf16":
        raise ValueError(kv_dtype)
    bits = f32.view(np.uint32).astype(np.uint64)
    # round the low 16 bits away, ties to the even upper half
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    top = (rounded & np.uint64(0xFFFF)).astype(np.uint16)
    return kv_to_f64(top, "bf16")


def page_moments(k_pool, block_table, seq_lens, page_size: int, kv_dtype: str):
    """Mean and population variance of the valid keys of every page in use,
    per KV head and coordinate, as stored: (mean, var) float64
    [P_phys, H_kv, D]; pages not used by any sequence stay NaN."""
    P_phys, Hkv, ps, D = k_pool.shape
    mean = np.full((P_phys, Hkv, D), np.nan)
    var = np.full((P_phys, Hkv, D), np.nan)
    for b in range(len(seq_lens)):
        for j in range(num_pages(seq_lens[b], page_size)):
            phys = int(block_table[b, j])
            nv = page_rows(j, seq_lens[b], page_size)
            rows = kv_to_f64(k_pool[phys, :, :nv, :], kv_dtype)  # [Hkv, nv, D]
            mean[phys] = round_to_kv(rows.mean(axis=1), kv_dtype)
            var[phys] = round_to_kv(rows.var(axis=1), kv_dtype)
    return mean, var


# ---------------------------------------------------------------------------
# [EntmaxKV page] section 2.B policy 2 (readings G2-G5)


def page_score_stats(q_h, mean_p, var_p, alpha: float):
    """(mu_a, s_a) of one page's scores in the units of tau (reading G2):
    mu_a = (alpha-1) q.mean, s_a = (alpha-1) sqrt((q*q).var)."""
    am1 = alpha_minus_one(alpha)
    q = np.asarray(q_h, dtype=np.float64)
    mu = float(np.dot(q, mean_p))
    s2 = float(np.dot(q * q, var_p))
    return am1 * mu, am1 * math.sqrt(max(s2, 0.0))


def alpha_minus_one(alpha: float) -> float:
    """alpha - 1 with alpha as the float32 the library receives."""
    return float(np.float32(alpha)) - 1.0


def integer_m(alpha: float) -> int:
    """m = 1/(alpha-1) for the supported alphas (2, 3/2, 4/3, 5/4 as float32)."""
    m = 1.0 / alpha_minus_one(alpha)
    r = round(m)
    if r < 1 or r > 4 or abs(m - r) > 1e-4:
        raise ValueError(f"alpha={alpha}: the Gaussian selection needs 1/(alpha-1) in 1..4")
    return int(r)


def normal_partial_moment(c, m: int):
    """E[(Y - c)_+^m] for Y ~ N(0, 1), integer m in 1..4, from the truncated
    moments J_k = E[Y^k; Y > c]: J_0 = Q(c), J_1 = phi(c),
    J_k = c^(k-1) phi(c) + (k-1) J_(k-2), and the binomial expansion of
    (Y - c)^m."""
    c = np.asarray(c, dtype=np.float64)
    phi = np.exp(-0.5 * c * c) / math.sqrt(2.0 * math.pi)
    J = [0.5 * erfc(c / math.sqrt(2.0)), phi]
    for k in range(2, m + 1):
        J.append(c ** (k - 1) * phi + (k - 1) * J[k - 2])
    total = sum(math.comb(m, k) * (-c) ** (m - k) * J[k] for k in range(m + 1))
    # The expansion cancels to rounding noise (|x| < 1e-300) where phi(c)
    # underflows, far in the right tail; the moment itself is never negative.
    return np.maximum(total, 0.0)


def expected_mass(t: float, mu_a, s_a, n, m: int) -> float:
    """Left side of the approximate normalisation (reading G3):
    sum_p n_p E[(A_p - t)_+^m], A_p ~ N(mu_a_p, s_a_p^2); a page with
    s_a = 0 contributes n_p (mu_a - t)_+^m exactly."""
    mu_a = np.asarray(mu_a, dtype=np.float64)
    s_a = np.asarray(s_a, dtype=np.float64)
    n = np.asarray(n, dtype=np.float64)
    total = 0.0
    point = s_a == 0.0
    if point.any():
        total += float(np.sum(n[point] * np.maximum(mu_a[point] - t, 0.0) ** m))
    spread = ~point
    if spread.any():
        c = (t - mu_a[spread]) / s_a[spread]
        total += float(np.sum(n[spread] * s_a[spread] ** m * normal_partial_moment(c, m)))
    return total


def gauss_threshold(mu_a, s_a, n, alpha: float) -> float:
    """tau_hat: root of expected_mass(t) = 1 by float64 bisection on
    [max mu_a - 1, max (mu_a + 40 s_a)] until the midpoint is an endpoint.
    At the left end the page with the largest mu_a alone contributes at least
    n_p (E[A_p] - t)^m = n_p >= 1 (Jensen: x_+^m is convex); at the right end
    every term is below 1e-300."""
    m = integer_m(alpha)
    mu_a = np.asarray(mu_a, dtype=np.float64)
    s_a = np.asarray(s_a, dtype=np.float64)
    lo = float(mu_a.max()) - 1.0
    hi = float((mu_a + 40.0 * s_a).max())
    if hi <= lo:
        hi = lo + 1.0
    assert expected_mass(lo, mu_a, s_a, n, m) >= 1.0
    assert expected_mass(hi, mu_a, s_a, n, m) < 1.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            return lo
        if expected_mass(mid, mu_a, s_a, n, m) >= 1.0:
            lo = mid
        else:
            hi = mid


def estimated_max(mu_a, s_a, n):
    """A page's estimated largest score in tau units (reading G4)."""
    mu_a = np.asarray(mu_a, dtype=np.float64)
    s_a = np.asarray(s_a, dtype=np.float64)
    n = np.asarray(n, dtype=np.float64)
    spread = np.sqrt(2.0 * np.log(np.maximum(n, 1.0)))
    return mu_a + s_a * spread


def gauss_select_pages(est, tau_hat: float, delta: float, cap: int) -> list:
    """Reading G5: pages with est > tau_hat - delta; at most `cap`, the largest
    float32 estimates first (ties to the lower page); ascending, -1 padded."""
    if cap <= 0:
        raise ValueError("cap must be positive")
    est = np.asarray(est, dtype=np.float64)
    passing = [j for j in range(len(est)) if est[j] > tau_hat - delta]
    if len(passing) > cap:
        key = est.astype(np.float32) + np.float32(0.0)
        passing = sorted(sorted(passing, key=lambda j: (-float(key[j]), j))[:cap])
    return passing + [-1] * (cap - len(passing))


def gauss_near_threshold(est, tau_hat: float, delta: float, cap: int,
                         rel: float = 1e-9, key_rel: float = 1e-6) -> set:
    """Pages whose selection may flip under float64 rounding of a different
    summation order: an estimate within rel of tau_hat - delta, or (when the
    cap binds) a float32 key within key_rel of the cap-th largest key."""
    est = np.asarray(est, dtype=np.float64)
    cut = tau_hat - delta
    tol = rel * max(1.0, abs(tau_hat))
    near = {j for j in range(len(est)) if abs(est[j] - cut) <= tol}
    passing = [j for j in range(len(est)) if est[j] > cut - tol]
    if len(passing) > cap:
        key = est.astype(np.float32).astype(np.float64)
        kth = float(np.sort(key[passing])[::-1][cap - 1])
        near |= {j for j in passing if abs(key[j] - kth) <= key_rel * abs(kth)}
    return near


def gauss_select_for_head(inp: dict, b: int, h: int, alpha: float, delta: float, cap: int,
                          moments=None):
    """Gaussian-aware selection of one (sequence, query head): returns
    (tau_hat, est [P_b], sel). `moments` is page_moments' output (computed
    here when omitted)."""
    w = inp["workload"]
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    if moments is None:
        moments = page_moments(inp["k_pool"], inp["block_table"], inp["seq_lens"], w.page_size,
                               w.kv_dtype)
    mean, var = moments
    L = int(inp["seq_lens"][b])
    P = num_pages(L, w.page_size)
    mu_a = np.empty(P)
    s_a = np.empty(P)
    n = np.empty(P)
    for j in range(P):
        phys = int(inp["block_table"][b, j])
        mu_a[j], s_a[j] = page_score_stats(inp["q"][b, h], mean[phys, g], var[phys, g], alpha)
        n[j] = page_rows(j, L, w.page_size)
    tau_hat = gauss_threshold(mu_a, s_a, n, alpha)
    est = estimated_max(mu_a, s_a, n)
    return tau_hat, est, gauss_select_pages(est, tau_hat, delta, cap)
