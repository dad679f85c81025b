"""Acceptance rule for index sets chosen from near-tied scores (test infrastructure).

With tau the k-th largest fp64 score of a row and eps = rel * |tau|, a candidate
set G of k distinct indices is valid iff it holds every index whose score is
above tau + eps and no index whose score is below tau - eps. Rows whose
k-th/(k+1)-th relative gap is at least ``rel`` therefore admit exactly one valid
set, the oracle's.
"""
from __future__ import annotations

import numpy as np


def valid_topk_sets(S: np.ndarray, G: np.ndarray, k: int, rel: float = 1e-6) -> np.ndarray:
    """Per row of S ([rows, N] fp64), whether G[row] (k indices) is a valid top-k set."""
    S = np.asarray(S, np.float64)
    G = np.asarray(G)
    rows, N = S.shape
    ok = np.zeros(rows, dtype=bool)
    for r in range(rows):
        g = G[r]
        if g.shape[0] != k or len(np.unique(g)) != k or g.min() < 0 or g.max() >= N:
            continue
        tau = np.sort(S[r])[::-1][k - 1]
        eps = rel * abs(tau)
        must = np.nonzero(S[r] > tau + eps)[0]
        allowed = S[r] >= tau - eps
        ok[r] = np.isin(must, g).all() and allowed[g].all()
    return ok


def valid_route_sets(R: np.ndarray, E: np.ndarray, s: int, rel: float = 1e-6) -> np.ndarray:
    """Same rule for the routed expert lists (order inside a list is not checked)."""
    return valid_topk_sets(R, E, s, rel)
