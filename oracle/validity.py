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
    G = np.asarray(G).astype(np.int64)
    rows, N = S.shape
    if G.shape != (rows, k):
        return np.zeros(rows, dtype=bool)
    in_range = ((G >= 0) & (G < N)).all(axis=1)
    Gc = np.clip(G, 0, N - 1)
    distinct = (np.diff(np.sort(Gc, axis=1), axis=1) != 0).all(axis=1) if k > 1 else np.ones(rows, bool)
    tau = -np.partition(-S, k - 1, axis=1)[:, k - 1]
    eps = rel * np.abs(tau)
    sg = np.take_along_axis(S, Gc, axis=1)
    allowed = (sg >= (tau - eps)[:, None]).all(axis=1)
    n_must = (S > (tau + eps)[:, None]).sum(axis=1)
    n_must_in = (sg > (tau + eps)[:, None]).sum(axis=1)
    return in_range & distinct & allowed & (n_must == n_must_in)


def valid_route_sets(R: np.ndarray, E: np.ndarray, s: int, rel: float = 1e-6) -> np.ndarray:
    """Same rule for the routed expert lists (order inside a list is not checked)."""
    return valid_topk_sets(R, E, s, rel)
