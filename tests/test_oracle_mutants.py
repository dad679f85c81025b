"""Planted mistakes in the oracle, on the CPU: each mutant must fail at least one
of the pins in test_oracle.py, which shows those pins constrain the oracle."""
import math

import numpy as np
import pytest

import oracle
from oracle import mita_oracle as mo
import test_oracle as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(mo, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _fails(*tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


def attend_scaled(scale_fn=None, drop_landmarks=False, landmark_values_from_v=False):
    def attend(Q, K, V, Qt, Vt, I, E, queries=None):
        Q, K, V, Qt, Vt = (np.asarray(x, np.float64) for x in (Q, K, V, Qt, Vt))
        N, d = Q.shape
        qs = range(N) if queries is None else list(queries)
        O = np.empty((len(qs), d))
        for row, q in enumerate(qs):
            keys = ([] if drop_landmarks else [Qt]) + [K[I[e]] for e in E[q]]
            lv = V[: Qt.shape[0]] if landmark_values_from_v else Vt
            vals = ([] if drop_landmarks else [lv]) + [V[I[e]] for e in E[q]]
            Ks, Vs = np.concatenate(keys), np.concatenate(vals)
            lg = (Ks @ Q[q]) * (scale_fn(d) if scale_fn else 1 / math.sqrt(d))
            w = np.exp(lg - lg.max())
            O[row] = (w / w.sum()) @ Vs
        return O
    return attend


OUTPUT_PINS = (pins.test_hand_worked_example,
               pins.test_k_equals_n_s_equals_1_is_full_attention_over_landmarks_and_keys,
               pins.test_k_equals_n_s_equals_m_adds_ln_m_to_key_logits)


def test_mutant_wrong_scale(monkeypatch):
    _patch(monkeypatch, "attend", attend_scaled(scale_fn=lambda d: 1.0 / d))
    assert _fails(*OUTPUT_PINS)


def test_mutant_missing_shared_expert(monkeypatch):
    _patch(monkeypatch, "attend", attend_scaled(drop_landmarks=True))
    assert _fails(*OUTPUT_PINS)


def test_mutant_landmark_values_not_shared_expert(monkeypatch):
    _patch(monkeypatch, "attend", attend_scaled(landmark_values_from_v=True))
    assert _fails(*OUTPUT_PINS)


def test_mutant_topk_ties_to_higher_index(monkeypatch):
    def topk(S, k):
        order = np.argsort(-S[:, ::-1], axis=1, kind="stable")
        return np.sort(S.shape[1] - 1 - order[:, :k], axis=1)
    _patch(monkeypatch, "topk_experts", topk)
    assert _fails(pins.test_topk_brute_force_with_ties)


def test_mutant_topk_smallest_scores(monkeypatch):
    _patch(monkeypatch, "topk_experts", lambda S, k: np.sort(np.argsort(S, axis=1, kind="stable")[:, :k], axis=1))
    assert _fails(pins.test_topk_matches_torch_topk_without_ties)


def test_mutant_scores_from_values(monkeypatch):
    orig_forward = mo.forward

    def forward(Q, K, V, *a, **kw):
        return orig_forward(Q, V, V, *a, **kw)   # transposed role: V used as keys
    monkeypatch.setattr(oracle, "forward", forward)
    assert _fails(pins.test_hand_worked_example, pins.test_single_landmark_is_mean_query,
                  pins.test_k_equals_n_s_equals_1_is_full_attention_over_landmarks_and_keys)


def test_mutant_pool_floor_windows(monkeypatch):
    _patch(monkeypatch, "adaptive_windows", lambda L, M: [((i * L) // M, ((i + 1) * L) // M) for i in range(M)])
    assert _fails(lambda: pins.test_pool_matches_torch_adaptive_avg_pool1d(100, 7),
                  pins.test_pool_windows_overlap_when_not_divisible)


def test_mutant_pool_column_major_landmarks(monkeypatch):
    orig = mo.pool

    def pool(Q, gh, gw, ph, pw):
        out = orig(Q, gh, gw, ph, pw)
        return out.reshape(ph, pw, -1).transpose(1, 0, 2).reshape(ph * pw, -1)
    _patch(monkeypatch, "pool", pool)
    assert _fails(lambda: pins.test_pool_matches_torch_adaptive_avg_pool2d(9, 13, 4, 5))


def test_mutant_route_ascending(monkeypatch):
    _patch(monkeypatch, "route", lambda Q, Qt, s, R=None: np.argsort(mo.route_scores(Q, Qt), axis=1, kind="stable")[:, :s])
    assert _fails(pins.test_route_brute_force_and_order, pins.test_hand_worked_example)


def test_mutant_shared_expert_unscaled(monkeypatch):
    def shared_expert(Qt, K, V):
        S = mo.scores(Qt, K)
        W = np.exp(S - S.max(axis=1, keepdims=True))
        return (W / W.sum(axis=1, keepdims=True)) @ V
    _patch(monkeypatch, "shared_expert", shared_expert)
    assert _fails(lambda: pins.test_shared_expert_matches_torch_sdpa(16, 1024, 64))


def _full_attention_mutant(scale=None, transpose_weights=False, keys_as_values=False):
    def full_attention(Q, K, V):
        Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
        d = Q.shape[1]
        lg = Q @ K.T * (scale(d) if scale else 1 / math.sqrt(d))
        W = np.exp(lg - lg.max(axis=1, keepdims=True))
        W = W / W.sum(axis=1, keepdims=True)
        if transpose_weights:
            W = W.T
        return W @ (K if keys_as_values else V)
    return full_attention


FULL_PINS = (lambda: pins.test_full_attention_matches_torch_sdpa(37, 16),
             pins.test_full_attention_brute_force, pins.test_full_attention_closed_forms)


@pytest.mark.parametrize("kw", [dict(scale=lambda d: 1.0 / d), dict(scale=lambda d: 1.0),
                                dict(transpose_weights=True), dict(keys_as_values=True)],
                         ids=["scale_1_over_d", "unscaled", "transposed_weights", "keys_as_values"])
def test_mutant_full_attention(monkeypatch, kw):
    _patch(monkeypatch, "full_attention", _full_attention_mutant(**kw))
    assert _fails(*FULL_PINS)


def test_full_attention_mutant_harness_is_faithful(monkeypatch):
    # the unmutated rewrite passes every pin, so a failure above is the mutation's
    _patch(monkeypatch, "full_attention", _full_attention_mutant())
    assert not _fails(*FULL_PINS)


MARGIN_PINS = (pins.test_topk_margins_hand_worked, pins.test_topk_margins_k_equals_n_is_inf,
               pins.test_route_margins_hand_worked, pins.test_margins_brute_force_random_rows)


def _margins_mutant(kind):
    def topk_margins(S, k):
        S = np.asarray(S, np.float64)
        N = S.shape[1]
        if kind == "zeros":
            return np.zeros(S.shape[0])
        if k >= N:
            return np.full(S.shape[0], np.inf)
        srt = -np.sort(-S, axis=1)
        if kind == "off_by_one":   # (k+1)-th and (k+2)-th instead of k-th and (k+1)-th
            a, b = srt[:, k], srt[:, min(k + 1, N - 1)]
        else:
            a, b = srt[:, k - 1], srt[:, k]
        if kind == "absolute":
            return a - b
        if kind == "wrong_denominator":   # divided by the (k+1)-th score
            return (a - b) / np.maximum(np.abs(b), 1e-300)
        return (a - b) / np.maximum(np.abs(a), 1e-300)
    return topk_margins


@pytest.mark.parametrize("kind", ["off_by_one", "absolute", "wrong_denominator", "zeros"])
def test_mutant_margins(monkeypatch, kind):
    fn = _margins_mutant(kind)
    _patch(monkeypatch, "topk_margins", fn)
    _patch(monkeypatch, "route_margins", lambda R, s: fn(R, s))
    assert _fails(*MARGIN_PINS)


def test_margins_mutant_harness_is_faithful(monkeypatch):
    fn = _margins_mutant("faithful")
    _patch(monkeypatch, "topk_margins", fn)
    _patch(monkeypatch, "route_margins", lambda R, s: fn(R, s))
    assert not _fails(*MARGIN_PINS)


# ---------------------------------------------------------------- backward
import test_oracle_backward as bpins

BACKWARD_PINS = (lambda: bpins.test_backward_matches_finite_differences(bpins.CASES[0]),
                 lambda: bpins.test_backward_matches_finite_differences(bpins.CASES[1]),
                 lambda: bpins.test_backward_matches_torch_autograd(bpins.CASES[1]),
                 bpins.test_value_gradient_mass_is_sum_of_output_gradients)


def _attend_backward_mutant(kind):
    def attend_backward(Q, K, V, Qt, Vt, I, E, dO):
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
            lg = (Ks @ Q[q]) * sc
            p = np.exp(lg - lg.max())
            p /= p.sum()
            O = p @ Vs
            dp = Vs @ dO[q]
            dl = p * (dO[q] @ O - dp) if kind == "sign" else p * (dp - dO[q] @ O)
            dQ[q] += (dl @ Ks) * (1.0 if kind == "dq_unscaled" else sc)
            dKs, dVs = np.outer(dl, Q[q]) * sc, np.outer(p, dO[q])
            dQt += dKs[:m]
            dVt += dVs[:m]
            if kind == "duplicates_dropped":   # fancy-index += keeps one contribution per token
                dK[toks] += dKs[m:]
                dV[toks] += dVs[m:]
            else:
                np.add.at(dK, toks, dKs[m:])
                np.add.at(dV, toks, dVs[m:])
        return dQ, dK, dV, dQt, dVt
    return attend_backward


@pytest.mark.parametrize("kind", ["sign", "dq_unscaled", "duplicates_dropped"])
def test_mutant_attend_backward(monkeypatch, kind):
    monkeypatch.setattr(mo, "attend_backward", _attend_backward_mutant(kind))
    assert _fails(*BACKWARD_PINS)


def test_mutant_backward_without_shared_expert_path(monkeypatch):
    monkeypatch.setattr(mo, "shared_expert_backward", lambda Qt, K, V, dVt: (0 * Qt, 0 * K, 0 * V))
    assert _fails(*BACKWARD_PINS)


def test_mutant_backward_without_pooling_path(monkeypatch):
    monkeypatch.setattr(mo, "pool_matrix", lambda N, gh, gw, ph, pw: np.zeros((ph * pw, N)))
    assert _fails(*BACKWARD_PINS)


def test_backward_mutant_harness_is_faithful(monkeypatch):
    monkeypatch.setattr(mo, "attend_backward", _attend_backward_mutant("faithful"))
    assert not _fails(*BACKWARD_PINS)
