"""Plain fp64 CPU oracle for the discarded probability mass of a kept set of
tokens, alpha-entmax against softmax (the comparison of the EntmaxKV page).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
report and CPU-baseline legs may import this module. The library (the HIP
path) never imports, links or runs it, and this module imports nothing from
the library.

Source: "Riepilogo Tecnico: EntmaxKV - Decodifica Consapevole del Supporto
per l'Attention Entmax" (gist.science, paper 2605.21649), [EntmaxKV page]:
  - section 3 (error bound): the output error ||o - o~|| is at most 2 B
    delta, with B a bound on the value vectors' norms and delta the total
    probability mass of the dropped tokens;
  - section 3 (support recovery): under softmax delta > 0 as soon as one
    token is dropped; under alpha-entmax delta = 0 when the kept set holds
    the support;
  - section 3 (comparison) and section 4 (quality of the approximation):
    under the same kept set alpha-entmax drops much less mass than softmax,
    and its relative output error goes to zero as the support is recovered.
Readings where the page is silent (M1-M3):
  M1  softmax is taken over the same scores z = q.k as alpha-entmax
      (temperature 1 on the stored, pre-scaled query; alpha-entmax tends to
      it as alpha -> 1);
  M2  the sparse softmax output renormalises the kept tokens' softmax
      weights (sum 1 over the kept set); the sparse alpha-entmax output
      re-solves tau over the kept set (as the decode does);
  M3  B is the largest value-vector norm among the head's tokens.
Every function works in float64. Pins: tests/test_oracle_mass.py.
"""
from __future__ import annotations

import numpy as np

from .entmax_oracle import entmax


def softmax(z) -> np.ndarray:
    """softmax(z)_i = exp(z_i - max z) / sum_j exp(z_j - max z)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def discarded_mass(p, keep) -> float:
    """delta: the probability mass of the tokens outside the kept set
    (keep: boolean mask over the same tokens as p)."""
    p = np.asarray(p, dtype=np.float64)
    keep = np.asarray(keep, dtype=bool)
    return float(p[~keep].sum())


def softmax_kept_output(z, V, keep) -> np.ndarray:
    """Sparse softmax output over the kept tokens (reading M2: the kept
    weights renormalised)."""
    keep = np.asarray(keep, dtype=bool)
    w = softmax(np.asarray(z, dtype=np.float64)[keep])
    return w @ np.asarray(V, dtype=np.float64)[keep]


def entmax_kept_output(z, V, keep, alpha: float) -> np.ndarray:
    """Sparse alpha-entmax output over the kept tokens (tau re-solved on
    them, reading M2)."""
    keep = np.asarray(keep, dtype=bool)
    p, _ = entmax(np.asarray(z, dtype=np.float64)[keep], alpha)
    return p @ np.asarray(V, dtype=np.float64)[keep]


def mass_comparison(z, V, keep, alpha: float) -> dict:
    """For one query over all of its tokens (scores z, values V) and a kept
    set: delta and the relative output error of alpha-entmax and of softmax,
    the kept fraction of the entmax support, and the section-3 bound 2 B
    delta for each (reading M3)."""
    z = np.asarray(z, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    keep = np.asarray(keep, dtype=bool)
    p_e, _ = entmax(z, alpha)
    p_s = softmax(z)
    o_e, o_s = p_e @ V, p_s @ V
    ot_e = entmax_kept_output(z, V, keep, alpha)
    ot_s = softmax_kept_output(z, V, keep)
    B = float(np.linalg.norm(V, axis=1).max())
    d_e, d_s = discarded_mass(p_e, keep), discarded_mass(p_s, keep)
    sup = p_e > 0
    return {
        "delta_entmax": d_e,
        "delta_softmax": d_s,
        "rel_err_entmax": float(np.linalg.norm(ot_e - o_e) / np.linalg.norm(o_e)),
        "rel_err_softmax": float(np.linalg.norm(ot_s - o_s) / np.linalg.norm(o_s)),
        "err_entmax": float(np.linalg.norm(ot_e - o_e)),
        "err_softmax": float(np.linalg.norm(ot_s - o_s)),
        "bound_entmax": 2.0 * B * d_e,
        "bound_softmax": 2.0 * B * d_s,
        "support": int(sup.sum()),
        "support_kept": int((sup & keep).sum()),
        "kept_tokens": int(keep.sum()),
        "tokens": int(len(z)),
    }
