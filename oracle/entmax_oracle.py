"""Plain fp64 CPU oracle for support-aware sparse alpha-entmax decode over a
paged KV cache (the EntmaxKV method).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module. The library (the HIP path) never
imports, links or runs it, and this module imports nothing from the library:
the two share only the seeded inputs produced by the synthetic generator.

Source of what is computed: "Riepilogo Tecnico: EntmaxKV - Decodifica
Consapevole del Supporto per l'Attention Entmax" (gist.science, paper
2605.21649), cited below as [EntmaxKV page]:
  - section 2, opening: alpha-entmax with alpha > 1 has exact zeros; if the
    kept tokens contain the support, the sparse output equals the full one;
  - section 2.A: the cache is split into pages, each page keeps a
    coordinate-wise bounding box (k_min, k_max) of its keys, which gives a
    deterministic upper bound on the best score of any token in the page;
  - section 2.B, policy 1: a fixed budget of the k pages with the highest
    bounds is selected;
  - section 2.C: only the selected pages' K/V are loaded and alpha-entmax is
    computed on that reduced set;
  - section 3: ||o - o~|| <= 2 B delta, and delta = 0 when the support is kept.
The pages never write the entmax formula. The definition used is the
standard Tsallis alpha-entmax of Peters, Niculae & Martins (ACL 2019):
    p_i = [(alpha-1) z_i - tau]_+ ^ (1/(alpha-1)),  tau chosen so sum p = 1,
equivalently p = argmax_{p in simplex} p.z + H_alpha(p) with the Tsallis
entropy H_alpha(p) = sum_j (p_j - p_j^alpha) / (alpha (alpha-1)).

Readings where the pages are silent:
  - the box bound is the maximum of q.k over the box:
    sum_d max(q_d kmin_d, q_d kmax_d);
  - scores are z = q.k on the stored values (no 1/sqrt(d) inside);
  - selection ranks the bound rounded once to float32, ties to the lower
    logical page index, the kept pages listed in ascending page order;
  - the sparse decode re-solves tau over the gathered tokens only;
  - only tokens t < seq_len are part of a page (partial last pages).

Every function works in float64 from the stored values (bf16 is widened
exactly). Parity pins for each function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# stored values -> float64


def kv_to_f64(arr: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Widen stored cache values exactly: bf16 bit patterns or float32."""
    if kv_dtype == "bf16":
        return (np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)
    if kv_dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


def num_pages(seq_len: int, page_size: int) -> int:
    return (int(seq_len) + page_size - 1) // page_size


def page_rows(j: int, seq_len: int, page_size: int) -> int:
    """Number of valid tokens in logical page j of a sequence of seq_len tokens."""
    return max(0, min(page_size, int(seq_len) - j * page_size))


# ---------------------------------------------------------------------------
# [EntmaxKV page] section 2.A: per-page bounding box metadata


def page_metadata(k_pool, block_table, seq_lens, page_size: int, kv_dtype: str):
    """Coordinate-wise min and max of the valid keys of every page in use.

    Returns (kmin, kmax), float64 [P_phys, H_kv, D]; pages not used by any
    sequence stay NaN. min/max are exact, so these are the stored values.
    """
    P_phys, Hkv, ps, D = k_pool.shape
    kmin = np.full((P_phys, Hkv, D), np.nan)
    kmax = np.full((P_phys, Hkv, D), np.nan)
    for b in range(len(seq_lens)):
        for j in range(num_pages(seq_lens[b], page_size)):
            phys = int(block_table[b, j])
            nv = page_rows(j, seq_lens[b], page_size)
            rows = kv_to_f64(k_pool[phys, :, :nv, :], kv_dtype)  # [Hkv, nv, D]
            kmin[phys] = rows.min(axis=1)
            kmax[phys] = rows.max(axis=1)
    return kmin, kmax


def sequence_metadata(k_pool, block_table_row, seq_len: int, page_size: int, g: int,
                      kv_dtype: str):
    """The boxes of every logical page of one sequence for KV head g, in
    logical page order: (kmin, kmax) float64 [P_b, D]. Same definition as
    page_metadata, restricted to one sequence."""
    P = num_pages(seq_len, page_size)
    D = k_pool.shape[-1]
    kmin = np.empty((P, D))
    kmax = np.empty((P, D))
    for j in range(P):
        phys = int(block_table_row[j])
        rows = kv_to_f64(k_pool[phys, g, :page_rows(j, seq_len, page_size), :], kv_dtype)
        kmin[j] = rows.min(axis=0)
        kmax[j] = rows.max(axis=0)
    return kmin, kmax


def page_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray) -> float:
    """Upper bound on q.k over the box [kmin, kmax] of one page (reading: the
    box maximum, sum_d max(q_d kmin_d, q_d kmax_d)).

    Each product of a float32 q with a bf16/float32 key is exact in float64;
    math.fsum returns the correctly rounded sum.
    """
    q = np.asarray(q, dtype=np.float64)
    terms = np.maximum(q * kmin, q * kmax)
    return math.fsum(terms.tolist())


def head_bounds(q_h, kmin, kmax, block_table_row, seq_len, page_size, g):
    """Bounds of every logical page j < P_b of one sequence for one query head."""
    P = num_pages(seq_len, page_size)
    out = np.empty(P)
    for j in range(P):
        phys = int(block_table_row[j])
        out[j] = page_bound(q_h, kmin[phys, g], kmax[phys, g])
    return out


def bound_key(ub: np.ndarray) -> np.ndarray:
    """The selection key: the bound rounded once to float32, -0 folded into +0."""
    return np.asarray(ub, dtype=np.float64).astype(np.float32) + np.float32(0.0)


# ---------------------------------------------------------------------------
# [EntmaxKV page] section 2.B policy 1: fixed-budget top-k pages


def select_pages(key32: np.ndarray, budget: int) -> list:
    """Top-`budget` logical pages by key, ties to the lower page index;
    returned ascending, padded with -1 to `budget` entries."""
    if budget <= 0:
        raise ValueError("budget must be positive")
    P = len(key32)
    order = sorted(range(P), key=lambda j: (-float(key32[j]), j))
    keep = sorted(order[:min(budget, P)])
    return keep + [-1] * (budget - len(keep))


def near_tie_pages(key32: np.ndarray, budget: int, rel: float = 1e-5) -> set:
    """Pages whose key lies within rel of the budget-th largest key. A GPU
    selection may differ from the oracle's only on such pages."""
    P = len(key32)
    if budget >= P:
        return set()
    kth = float(np.sort(np.asarray(key32, dtype=np.float64))[::-1][budget - 1])
    tol = rel * abs(kth)
    return {j for j in range(P) if abs(float(key32[j]) - kth) <= tol}


# ---------------------------------------------------------------------------
# alpha-entmax threshold (Peters, Niculae & Martins 2019), three ways


def _power(x: np.ndarray, m: float) -> np.ndarray:
    return np.power(x, m)


def entmax_threshold(a: np.ndarray, alpha: float) -> float:
    """Exact tau for sum_i [a_i - tau]_+^m = 1, m = 1/(alpha-1), by sorting.

    Only a_i > max(a) - 1 can be in the support (at tau = max(a) - 1 the top
    term alone is 1), so the search is restricted to that window. In
    descending order c_1 >= c_2 >= ..., the support is the top k* where k* is
    the largest k with sum_{j<k} (c_j - c_k)^m < 1; tau then solves the
    equation on those k* values: closed form for m = 1 and m = 2, bisection
    to the float64 fixed point otherwise.
    """
    a = np.asarray(a, dtype=np.float64)
    if a.size == 0:
        raise ValueError("empty score vector")
    m = 1.0 / (alpha - 1.0)
    amax = float(a.max())
    c = np.sort(a[a > amax - 1.0])[::-1]
    n = len(c)

    def gap_sum(k: int) -> float:  # k is 1-based
        return float(_power(c[:k - 1] - c[k - 1], m).sum())

    lo_k, hi_k = 1, n  # gap_sum(1) = 0 < 1
    while lo_k < hi_k:
        mid = (lo_k + hi_k + 1) // 2
        if gap_sum(mid) < 1.0:
            lo_k = mid
        else:
            hi_k = mid - 1
    k = lo_k
    top = c[:k]
    if m == 1.0:
        return float((top.sum() - 1.0) / k)
    if m == 2.0:
        mu = float(top.mean())
        cvar = float(((top - mu) ** 2).sum())
        return mu - math.sqrt((1.0 - cvar) / k)
    lo = max(amax - 1.0, float(c[k]) if k < n else amax - 1.0)
    hi = float(c[k - 1])
    for _ in range(10000):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if float(_power(top - mid, m).sum()) >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def entmax_threshold_bisect(a: np.ndarray, alpha: float) -> float:
    """tau by plain bisection over all a on [max(a) - 1, max(a) - n^(1-alpha)]
    (at the left end the top term alone is 1, at the right end every term is
    at most 1/n), run to the float64 fixed point."""
    a = np.asarray(a, dtype=np.float64)
    m = 1.0 / (alpha - 1.0)
    n = a.size
    amax = float(a.max())
    lo, hi = amax - 1.0, amax - n ** (-(alpha - 1.0))
    for _ in range(10000):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        f = float(_power(np.maximum(a - mid, 0.0), m).sum())
        if f >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def entmax_threshold_bruteforce(a: np.ndarray, alpha: float):
    """tau and support by enumerating every non-empty subset S (n <= 14):
    solve sum_{i in S} (a_i - tau)^m = 1 for tau < min a_S and keep the S
    whose tau splits a into S (a_i > tau) and the rest (a_i <= tau)."""
    a = np.asarray(a, dtype=np.float64)
    n = a.size
    if n > 14:
        raise ValueError("brute force is for tiny inputs")
    m = 1.0 / (alpha - 1.0)
    found = []
    for mask in range(1, 1 << n):
        S = [i for i in range(n) if mask >> i & 1]
        aS = a[S]
        lo, hi = float(aS.max()) - 1.0, float(aS.min())
        if float(_power(aS - hi, m).sum()) >= 1.0:
            continue  # no root below min a_S
        for _ in range(10000):
            mid = 0.5 * (lo + hi)
            if mid <= lo or mid >= hi:
                break
            if float(_power(aS - mid, m).sum()) >= 1.0:
                lo = mid
            else:
                hi = mid
        tau = 0.5 * (lo + hi)
        inside = all(a[i] > tau for i in S)
        outside = all(a[i] <= tau + 1e-12 for i in range(n) if i not in S)
        if inside and outside:
            found.append((tau, tuple(S)))
    if not found:
        raise RuntimeError("no consistent support found")
    # Rounding can make two supports that differ only in a token sitting on
    # the boundary both look consistent; they share tau to rounding.
    found.sort(key=lambda t: len(t[1]))
    return found[0]


def entmax_probs(a: np.ndarray, tau: float, alpha: float) -> np.ndarray:
    """p_i = [a_i - tau]_+^m; a token exactly at tau gets 0 (no renormalisation)."""
    a = np.asarray(a, dtype=np.float64)
    m = 1.0 / (alpha - 1.0)
    d = a - tau
    p = np.zeros_like(a)
    pos = d > 0
    p[pos] = _power(d[pos], m)
    return p


def entmax(z: np.ndarray, alpha: float):
    """alpha-entmax of scores z: returns (p, tau) with tau in the (alpha-1) z units."""
    a = (alpha - 1.0) * np.asarray(z, dtype=np.float64)
    tau = entmax_threshold(a, alpha)
    return entmax_probs(a, tau, alpha), tau


# ---------------------------------------------------------------------------
# gathering tokens of a sequence ([EntmaxKV page] section 2.C)


def gather_tokens(pool, b: int, g: int, block_table, seq_lens, page_size: int,
                  kv_dtype: str, pages=None):
    """Valid tokens of the listed logical pages (all pages if None), in
    ascending token order, as float64 [n, D], with their token positions."""
    L = int(seq_lens[b])
    P = num_pages(L, page_size)
    if pages is None:
        pages = range(P)
    pages = [int(j) for j in pages if j >= 0]
    rows, pos = [], []
    for j in sorted(pages):
        if j >= P:
            raise ValueError("page beyond the sequence")
        nv = page_rows(j, L, page_size)
        phys = int(block_table[b, j])
        rows.append(kv_to_f64(pool[phys, g, :nv, :], kv_dtype))
        pos.extend(range(j * page_size, j * page_size + nv))
    D = pool.shape[-1]
    if not rows:
        return np.zeros((0, D)), np.zeros(0, dtype=np.int64)
    return np.concatenate(rows), np.asarray(pos, dtype=np.int64)


@dataclass
class DecodeResult:
    out: np.ndarray  # [D] float64
    tau: float
    support: int
    support_pos: np.ndarray  # token positions with p > 0
    probs: np.ndarray  # over the gathered tokens
    positions: np.ndarray  # token positions of the gathered tokens
    scores: np.ndarray


def decode_tokens(q_h, K, V, positions, alpha: float) -> DecodeResult:
    """alpha-entmax attention of one query over the given tokens: o = sum p v."""
    q = np.asarray(q_h, dtype=np.float64)
    if K.shape[0] == 0:
        D = q.shape[0]
        return DecodeResult(np.zeros(D), float("nan"), 0, np.zeros(0, np.int64),
                            np.zeros(0), positions, np.zeros(0))
    z = K @ q
    p, tau = entmax(z, alpha)
    out = p @ V
    nz = p > 0
    return DecodeResult(out, tau, int(nz.sum()), positions[nz], p, positions, z)


def decode_full(inp: dict, b: int, h: int, alpha: float) -> DecodeResult:
    """Full-cache alpha-entmax decode of query head h of sequence b."""
    w = inp["workload"]
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    K, pos = gather_tokens(inp["k_pool"], b, g, inp["block_table"], inp["seq_lens"],
                           w.page_size, w.kv_dtype)
    V, _ = gather_tokens(inp["v_pool"], b, g, inp["block_table"], inp["seq_lens"],
                         w.page_size, w.kv_dtype)
    return decode_tokens(inp["q"][b, h], K, V, pos, alpha)


def decode_sparse(inp: dict, b: int, h: int, alpha: float, sel) -> DecodeResult:
    """alpha-entmax decode of head h of sequence b over the pages in `sel`
    (logical page indices, -1 entries ignored); tau is re-solved on them."""
    w = inp["workload"]
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    K, pos = gather_tokens(inp["k_pool"], b, g, inp["block_table"], inp["seq_lens"],
                           w.page_size, w.kv_dtype, pages=sel)
    V, _ = gather_tokens(inp["v_pool"], b, g, inp["block_table"], inp["seq_lens"],
                         w.page_size, w.kv_dtype, pages=sel)
    return decode_tokens(inp["q"][b, h], K, V, pos, alpha)


def select_for_head(inp: dict, b: int, h: int, budget: int, meta=None, seq_meta=None):
    """Bounds and selection of one head: returns (ub float64 [P_b], key32, sel).
    `meta` is page_metadata's output; `seq_meta` is sequence_metadata's for
    this (sequence, KV head); with neither, the boxes are computed here."""
    w = inp["workload"]
    G = w.num_q_heads // w.num_kv_heads
    g = h // G
    q = inp["q"][b, h].astype(np.float64)
    if seq_meta is None and meta is None:
        seq_meta = sequence_metadata(inp["k_pool"], inp["block_table"][b], inp["seq_lens"][b],
                                     w.page_size, g, w.kv_dtype)
    if seq_meta is not None:
        kmin, kmax = seq_meta
        ub = np.array([page_bound(q, kmin[j], kmax[j]) for j in range(kmin.shape[0])])
    else:
        kmin, kmax = meta
        ub = head_bounds(q, kmin, kmax, inp["block_table"][b], inp["seq_lens"][b], w.page_size, g)
    key = bound_key(ub)
    return ub, key, select_pages(key, budget)


def support_pages(result: DecodeResult, page_size: int) -> list:
    """Logical pages holding the support of a decode result."""
    return sorted(set(int(t) // page_size for t in result.support_pos))
