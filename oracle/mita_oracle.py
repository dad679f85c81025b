"""Plain fp64 reference of the MiTA attention forward pass, one (batch, head) slice.

TEST INFRASTRUCTURE. Imported only by ``tests/``, the smoke check and the CPU
baseline of the benchmark; the GPU product path never reaches it.

Source: the three summaries of "MiTA Attention: Efficient Fast-Weight Scaling via
a Mixture of Top-k Activations" on gist.science (Arabic, Dutch and Hindi pages).
Each function names the section it follows. Every value is float64; bf16 or
fp32 inputs are widened exactly before use. numpy's matmul, sort and exp are the
only library steps; nothing is blocked, fused or reordered beyond what the
method states.

Readings taken where the pages leave a step open (all follow the plainest
reading consistent with the rest):
  * the pooling is adaptive average pooling with the usual window rule
    start = floor(i L / M), end = ceil((i + 1) L / M), per axis; 2D workloads
    pool a row-major token grid separably, landmarks numbered row-major;
  * Atten(.) is softmax attention with scale 1/sqrt(d), used both for the
    shared expert and for the final attention;
  * the landmark queries are also the keys of the shared expert, the landmark
    values its values;
  * expert i is the k largest raw scores q~_i . K_n over all N tokens; ties
    go to the lower token index; the index list is reported ascending;
  * a query is routed to the s landmarks with the largest q . q~_i (ties to
    the lower landmark index), listed by descending score;
  * the final key list is the concatenation as written, so a token that sits in
    two of a query's experts appears twice;
  * no mask of any kind.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np


def adaptive_windows(L: int, M: int):
    """Window [start, end) of each of M adaptive-average-pooling cells over L
    positions (landmark construction by adaptive average pooling: Arabic and
    Hindi summaries, section 2 "mechanism details"; Dutch summary, "Kernconcepten"
    item 1)."""
    return [((i * L) // M, -((-(i + 1) * L) // M)) for i in range(M)]


def pool(Q: np.ndarray, grid_h: int, grid_w: int, pool_h: int, pool_w: int) -> np.ndarray:
    """Landmark queries Q~ [m, d]: the mean of Q over each pooling cell.

    Q is [N, d] with N = grid_h * grid_w tokens in row-major grid order
    (grid_h = 1 for a 1D sequence). Landmark ids are row-major over the
    pool_h x pool_w cell grid. Follows the landmark-query construction of
    the summaries' method sections (down-sampling Q by average pooling).
    """
    Q = np.asarray(Q, dtype=np.float64)
    N, d = Q.shape
    assert N == grid_h * grid_w
    G = Q.reshape(grid_h, grid_w, d)
    out = np.empty((pool_h * pool_w, d), dtype=np.float64)
    for a, (r0, r1) in enumerate(adaptive_windows(grid_h, pool_h)):
        for b, (c0, c1) in enumerate(adaptive_windows(grid_w, pool_w)):
            cell = G[r0:r1, c0:c1].reshape(-1, d)
            out[a * pool_w + b] = cell.sum(axis=0) / cell.shape[0]
    return out


def scores(Qt: np.ndarray, K: np.ndarray) -> np.ndarray:
    """Raw activations K q~_i for every landmark i and token n: [m, N]
    (deformable experts: Arabic/Hindi section 2; Dutch "Kernconcepten" item 3)."""
    return np.asarray(Qt, np.float64) @ np.asarray(K, np.float64).T


def _softmax_rows(x: np.ndarray) -> np.ndarray:
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def shared_expert(Qt: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Shared expert V~ = Atten(Q~, K, V) = softmax(Q~ K^T / sqrt d) V, [m, d]
    (compression step: Arabic/Hindi section 2 "core concept" and "mechanism
    details"; Dutch "Kernconcepten" item 2)."""
    d = Qt.shape[1]
    W = _softmax_rows(scores(Qt, K) / math.sqrt(d))
    return W @ np.asarray(V, np.float64)


def full_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Standard softmax attention over all N keys, softmax(Q K^T / sqrt d) V,
    [N, d]: the quadratic-cost baseline the pages set MiTA against (Arabic/Hindi
    section 1 and the Dutch "Probleemstelling"). Not a step of MiTA."""
    d = Q.shape[1]
    W = _softmax_rows(np.asarray(Q, np.float64) @ np.asarray(K, np.float64).T / math.sqrt(d))
    return W @ np.asarray(V, np.float64)


def topk_experts(S: np.ndarray, k: int) -> np.ndarray:
    """Expert index sets I_i: the k tokens with the largest S[i, n], ties to the
    lower n, listed ascending; [m, k] int64 (top-k activations of K^T q~_i:
    Arabic/Hindi section 2; Dutch "Wiskundige Formulering")."""
    order = np.argsort(-S, axis=1, kind="stable")   # by (-score, index)
    return np.sort(order[:, :k], axis=1)


def route_scores(Q: np.ndarray, Qt: np.ndarray) -> np.ndarray:
    """Router activations q . q~_i for every query and landmark: [N, m]."""
    return np.asarray(Q, np.float64) @ np.asarray(Qt, np.float64).T


def route(Q: np.ndarray, Qt: np.ndarray, s: int, R: Optional[np.ndarray] = None) -> np.ndarray:
    """Routed experts e_1(q) .. e_s(q) of each query: the s landmarks with the
    largest q . q~_i, ties to the lower landmark id, by descending score; [N, s]
    (routing of a query to a subset of experts: Arabic/Hindi section 2 and the
    Dutch "Wiskundige Formulering"; the pages do not state the rule, this
    dot-product top-s is the reading taken)."""
    if R is None:
        R = route_scores(Q, Qt)
    return np.argsort(-R, axis=1, kind="stable")[:, :s]


def attend(Q, K, V, Qt, Vt, I, E, queries: Optional[Sequence[int]] = None) -> np.ndarray:
    """Final output for each query q (all when ``queries`` is None): softmax
    attention of q over K* = [Q~, K^(e_1(q)), ..., K^(e_s(q))] with values
    V* = [V~, V^(e_1(q)), ..., V^(e_s(q))], scale 1/sqrt(d), duplicates kept
    (Dutch summary, "Wiskundige Formulering"; Arabic/Hindi section 2,
    attention computation)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Qt = np.asarray(Qt, np.float64)
    Vt = np.asarray(Vt, np.float64)
    N, d = Q.shape
    qs = range(N) if queries is None else list(queries)
    O = np.empty((len(qs), d), dtype=np.float64)
    for row, q in enumerate(qs):
        keys = [Qt] + [K[I[e]] for e in E[q]]
        vals = [Vt] + [V[I[e]] for e in E[q]]
        Ks = np.concatenate(keys, axis=0)
        Vs = np.concatenate(vals, axis=0)
        logits = (Ks @ Q[q]) / math.sqrt(d)
        w = np.exp(logits - logits.max())
        w /= w.sum()
        O[row] = w @ Vs
    return O


def topk_margins(S: np.ndarray, k: int) -> np.ndarray:
    """Relative gap (s_(k) - s_(k+1)) / max(|s_(k)|, 1e-300) per row; +inf when k == N."""
    N = S.shape[1]
    if k >= N:
        return np.full(S.shape[0], np.inf)
    srt = -np.sort(-S, axis=1)
    a, b = srt[:, k - 1], srt[:, k]
    return (a - b) / np.maximum(np.abs(a), 1e-300)


def route_margins(R: np.ndarray, s: int) -> np.ndarray:
    """Relative gap between the s-th and (s+1)-th router score per query."""
    return topk_margins(R, s)


def forward(Q, K, V, grid_h: int, grid_w: int, pool_h: int, pool_w: int, k: int, s: int,
            queries: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """All five steps on one slice: pool, shared expert, expert sets, routing and
    the output (for ``queries`` only when given). Returns the intermediates too."""
    Qt = pool(Q, grid_h, grid_w, pool_h, pool_w)
    S = scores(Qt, K)
    Vt = shared_expert(Qt, K, V)
    I = topk_experts(S, k)
    R = route_scores(Q, Qt) if queries is None else None
    if queries is None:
        E = route(Q, Qt, s, R)
    else:
        # routing is needed only for the requested queries
        E_part = route(np.asarray(Q, np.float64)[list(queries)], Qt, s)
        E = np.full((np.asarray(Q).shape[0], s), -1, dtype=np.int64)
        E[list(queries)] = E_part
    O = attend(Q, K, V, Qt, Vt, I, E, queries)
    return {"Qt": Qt, "S": S, "Vt": Vt, "I": I, "E": E, "O": O, "R": R}


# ---------------------------------------------------------------- backward
# Gradients of the forward pass above with respect to Q, K and V, the expert sets
# I and the routing E held fixed (they are selections, not differentiable). The
# Long Range Arena training result on the MiTA pages (Arabic/Hindi section 4,
# Dutch "Resultaten") implies training through this operator; the pages give no
# backward, so this is the derivative of the forward as defined, by the chain
# rule, written out step by step.

def pool_matrix(N: int, grid_h: int, grid_w: int, pool_h: int, pool_w: int) -> np.ndarray:
    """The pooling as a matrix P [m, N]: Q~ = P Q, row i holding 1/|window i| on
    the window's tokens (the landmark construction of the method sections)."""
    P = np.zeros((pool_h * pool_w, N), dtype=np.float64)
    for a, (r0, r1) in enumerate(adaptive_windows(grid_h, pool_h)):
        for b, (c0, c1) in enumerate(adaptive_windows(grid_w, pool_w)):
            toks = [r * grid_w + c for r in range(r0, r1) for c in range(c0, c1)]
            P[a * pool_w + b, toks] = 1.0 / len(toks)
    return P


def attend_backward(Q, K, V, Qt, Vt, I, E, dO):
    """Backward of `attend` (the final attention over [Q~, K^(e_1(q)), ...] with
    values [V~, V^(e_1(q)), ...], Dutch "Wiskundige Formulering"): for each query,
    with p its attention weights and O its output, dp_j = dO . v*_j, the logit
    gradient is p_j (dp_j - dO . O), and it flows to q (times k*_j / sqrt d), to
    each key k*_j (times q / sqrt d) and, through p, to each value v*_j (p_j dO).
    A token present in two of the query's experts receives both contributions.
    Returns dQ (direct part), dK, dV (routed part), dQt, dVt."""
    Q, K, V, Qt, Vt, dO = (np.asarray(x, np.float64) for x in (Q, K, V, Qt, Vt, dO))
    N, d = Q.shape
    m = Qt.shape[0]
    sc = 1.0 / math.sqrt(d)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dQt, dVt = np.zeros_like(Qt), np.zeros_like(Vt)
    for q in range(N):
        toks = np.concatenate([np.asarray(I[e], dtype=np.int64) for e in E[q]])
        Ks = np.concatenate([Qt, K[toks]], axis=0)
        Vs = np.concatenate([Vt, V[toks]], axis=0)
        logits = (Ks @ Q[q]) * sc
        p = np.exp(logits - logits.max())
        p /= p.sum()
        O = p @ Vs
        dp = Vs @ dO[q]
        dl = p * (dp - dO[q] @ O)
        dQ[q] += (dl @ Ks) * sc
        dKs = np.outer(dl, Q[q]) * sc
        dVs = np.outer(p, dO[q])
        dQt += dKs[:m]
        dVt += dVs[:m]
        np.add.at(dK, toks, dKs[m:])
        np.add.at(dV, toks, dVs[m:])
    return dQ, dK, dV, dQt, dVt


def shared_expert_backward(Qt, K, V, dVt):
    """Backward of V~ = softmax(Q~ K^T / sqrt d) V (the shared expert, Arabic/Hindi
    section 2): with A the weights, dA = dV~ V^T, the score gradient is
    A (dA - rowsum(A dA)), and it flows to Q~ (times K / sqrt d) and to K (times
    Q~ / sqrt d); V gets A^T dV~. Returns dQt, dK, dV."""
    Qt, K, V, dVt = (np.asarray(x, np.float64) for x in (Qt, K, V, dVt))
    d = Qt.shape[1]
    sc = 1.0 / math.sqrt(d)
    A = _softmax_rows(scores(Qt, K) * sc)
    dA = dVt @ V.T
    dS = A * (dA - (A * dA).sum(axis=1, keepdims=True))
    return (dS @ K) * sc, (dS.T @ Qt) * sc, A.T @ dVt


def backward(Q, K, V, grid_h: int, grid_w: int, pool_h: int, pool_w: int, I, E, dO) -> Dict[str, np.ndarray]:
    """Gradients (dQ, dK, dV) of sum(dO * O) for the forward pass on one slice, with
    the expert sets I and routing E held fixed. Chain: the final attention, then
    the shared expert (its V~ feeds the final attention; Q~ is both its query and
    a key of the final attention), then the pooling (dQ += P^T dQ~)."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    N = Q.shape[0]
    Qt = pool(Q, grid_h, grid_w, pool_h, pool_w)
    Vt = shared_expert(Qt, K, V)
    dQ, dK, dV, dQt, dVt = attend_backward(Q, K, V, Qt, Vt, I, E, dO)
    dQt2, dK2, dV2 = shared_expert_backward(Qt, K, V, dVt)
    dQt = dQt + dQt2
    dQ = dQ + pool_matrix(N, grid_h, grid_w, pool_h, pool_w).T @ dQt
    return {"dQ": dQ, "dK": dK + dK2, "dV": dV + dV2, "dQt": dQt, "dVt": dVt}
