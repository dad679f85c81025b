"""Pins of the fp64 oracle against things other than itself: closed forms,
library routines on special cases, brute force on tiny inputs and invariants of
the method. CPU only."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

torch.set_default_dtype(torch.float64)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- pooling

def test_pool_closed_form_1d_divisible():
    # Q[n, c] = n + 1000 c: the mean over [a, b) is (a + b - 1) / 2 + 1000 c
    N, d, m = 64, 3, 8
    Q = np.arange(N)[:, None] + 1000.0 * np.arange(d)[None, :]
    Qt = oracle.pool(Q, 1, N, 1, m)
    for i in range(m):
        a, b = i * N // m, (i + 1) * N // m
        np.testing.assert_array_equal(Qt[i], (a + b - 1) / 2 + 1000.0 * np.arange(d))


def test_pool_windows_overlap_when_not_divisible():
    # adaptive windows for L=10, M=4: [0,3) [2,5) [5,8) [7,10)
    assert oracle.adaptive_windows(10, 4) == [(0, 3), (2, 5), (5, 8), (7, 10)]
    assert oracle.adaptive_windows(7, 7) == [(i, i + 1) for i in range(7)]
    assert oracle.adaptive_windows(5, 1) == [(0, 5)]


@pytest.mark.parametrize("N,m", [(64, 8), (100, 7), (33, 33), (17, 1), (1024, 16)])
def test_pool_matches_torch_adaptive_avg_pool1d(N, m):
    Q = rand((N, 5), N * m)
    ref = F.adaptive_avg_pool1d(torch.from_numpy(Q.T[None]), m)[0].numpy().T
    np.testing.assert_allclose(oracle.pool(Q, 1, N, 1, m), ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("gh,gw,ph,pw", [(56, 56, 8, 8), (16, 16, 4, 4), (9, 13, 4, 5), (6, 10, 6, 1)])
def test_pool_matches_torch_adaptive_avg_pool2d(gh, gw, ph, pw):
    d = 4
    Q = rand((gh * gw, d), gh * gw + ph)
    img = torch.from_numpy(Q.reshape(gh, gw, d).transpose(2, 0, 1).copy())[None]   # [1, d, gh, gw]
    ref = F.adaptive_avg_pool2d(img, (ph, pw))[0].numpy()                       # [d, ph, pw]
    ref = ref.transpose(1, 2, 0).reshape(ph * pw, d)                            # row-major landmarks
    np.testing.assert_allclose(oracle.pool(Q, gh, gw, ph, pw), ref, rtol=1e-14, atol=1e-14)


def test_pool_identity_and_mean():
    Q = rand((20, 3), 1)
    np.testing.assert_array_equal(oracle.pool(Q, 1, 20, 1, 20), Q)
    np.testing.assert_allclose(oracle.pool(Q, 4, 5, 1, 1)[0], Q.mean(axis=0), rtol=1e-14)


# ---------------------------------------------------------------- shared expert

def test_shared_expert_brute_force_loops():
    m, N, d = 3, 7, 4
    Qt, K, V = rand((m, d), 2), rand((N, d), 3), rand((N, d), 4)
    got = oracle.shared_expert(Qt, K, V)
    for i in range(m):
        logits = [sum(Qt[i, c] * K[n, c] for c in range(d)) / math.sqrt(d) for n in range(N)]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        for c in range(d):
            assert abs(got[i, c] - sum(w[n] * V[n, c] for n in range(N)) / z) < 1e-13


@pytest.mark.parametrize("m,N,d", [(16, 1024, 64), (5, 33, 128)])
def test_shared_expert_matches_torch_sdpa(m, N, d):
    Qt, K, V = rand((m, d), 5), rand((N, d), 6) * 2, rand((N, d), 7)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x)[None, None] for x in (Qt, K, V)))[0, 0].numpy()
    np.testing.assert_allclose(oracle.shared_expert(Qt, K, V), ref, rtol=1e-12, atol=1e-12)


def test_shared_expert_weights_sum_to_one():
    Qt, K = rand((6, 8), 8) * 3, rand((50, 8), 9) * 3
    np.testing.assert_allclose(oracle.shared_expert(Qt, K, np.ones((50, 8))), 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- top-k experts

def brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda n: (-row[n], n))
    return sorted(order[:k])


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(10)
    S = rng.integers(-3, 4, size=(20, 15)).astype(np.float64)   # many exact ties
    for k in (1, 4, 15):
        I = oracle.topk_experts(S, k)
        for i in range(S.shape[0]):
            assert list(I[i]) == brute_topk(list(S[i]), k)


def test_topk_matches_torch_topk_without_ties():
    S = rand((12, 3136), 11)
    I = oracle.topk_experts(S, 64)
    ref = torch.topk(torch.from_numpy(S), 64, dim=1).indices.numpy()
    np.testing.assert_array_equal(I, np.sort(ref, axis=1))


def test_topk_scores_use_keys_and_landmarks():
    # expert sets come from K q~_i, not from V or from the raw queries
    Q, K, V = rand((40, 6), 12), rand((40, 6), 13), rand((40, 6), 14)
    Qt = oracle.pool(Q, 1, 40, 1, 4)
    I = oracle.topk_experts(oracle.scores(Qt, K), 5)
    for i in range(4):
        row = [float(np.dot(Qt[i], K[n])) for n in range(40)]
        assert list(I[i]) == brute_topk(row, 5)


def test_topk_k_equals_n_selects_everything():
    S = rand((3, 9), 15)
    np.testing.assert_array_equal(oracle.topk_experts(S, 9), np.tile(np.arange(9), (3, 1)))


# ---------------------------------------------------------------- routing

def test_route_brute_force_and_order():
    rng = np.random.default_rng(16)
    Q = rng.integers(-2, 3, size=(30, 3)).astype(np.float64)
    Qt = rng.integers(-2, 3, size=(6, 3)).astype(np.float64)
    for s in (1, 2, 6):
        E = oracle.route(Q, Qt, s)
        for q in range(30):
            r = [float(np.dot(Q[q], Qt[i])) for i in range(6)]
            assert list(E[q]) == sorted(range(6), key=lambda i: (-r[i], i))[:s]


def test_route_s_equals_m_uses_all_experts():
    Q, Qt = rand((25, 4), 17), rand((5, 4), 18)
    E = oracle.route(Q, Qt, 5)
    np.testing.assert_array_equal(np.sort(E, axis=1), np.tile(np.arange(5), (25, 1)))


# ---------------------------------------------------------------- output

def brute_output(Q, K, V, Qt, Vt, I, E):
    """Explicit K*, V* lists and a pure-Python softmax, one query at a time."""
    N, d = Q.shape
    out = np.zeros((N, d))
    for q in range(N):
        keys = [Qt[j] for j in range(Qt.shape[0])]
        vals = [Vt[j] for j in range(Vt.shape[0])]
        for e in E[q]:
            for t in I[e]:
                keys.append(K[t])
                vals.append(V[t])
        logits = [sum(Q[q, c] * kk[c] for c in range(d)) / math.sqrt(d) for kk in keys]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        for c in range(d):
            out[q, c] = sum(wi * vv[c] for wi, vv in zip(w, vals)) / z
    return out


@pytest.mark.parametrize("N,d,m,k,s", [(16, 4, 4, 3, 1), (24, 3, 6, 5, 2), (12, 2, 3, 12, 3)])
def test_attend_brute_force(N, d, m, k, s):
    Q, K, V = rand((N, d), N), rand((N, d), N + 1), rand((N, d), N + 2)
    r = oracle.forward(Q, K, V, 1, N, 1, m, k, s)
    # brute force rebuilds every intermediate from the definitions
    Qt = np.array([[sum(Q[n, c] for n in range(a, b)) / (b - a) for c in range(d)]
                   for a, b in [(i * N // m, -(-(i + 1) * N // m)) for i in range(m)]])
    S = [[sum(Qt[i, c] * K[n, c] for c in range(d)) for n in range(N)] for i in range(m)]
    I = [brute_topk(S[i], k) for i in range(m)]
    E = [sorted(range(m), key=lambda i: (-float(np.dot(Q[q], Qt[i])), i))[:s] for q in range(N)]
    Vt = np.zeros((m, d))
    for i in range(m):
        w = [math.exp(S[i][n] / math.sqrt(d) - max(S[i]) / math.sqrt(d)) for n in range(N)]
        Vt[i] = sum(w[n] * V[n] for n in range(N)) / sum(w)
    np.testing.assert_allclose(r["Qt"], Qt, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["Vt"], Vt, rtol=1e-12, atol=1e-13)
    assert [list(x) for x in r["I"]] == I
    assert [list(x) for x in r["E"]] == E
    np.testing.assert_allclose(r["O"], brute_output(Q, K, V, Qt, Vt, I, E), rtol=1e-12, atol=1e-13)


def test_hand_worked_example():
    """Four tokens, d = 2, two landmarks, k = s = 1, values worked out by hand.

    Q~ = [[1,0],[0,1]]; landmark 0's scaled logits are [ln2,0,0,0] -> weights
    [2,1,1,1]/5 -> V~0 = [4,3]; landmark 1's are [0,0,ln2,0] -> V~1 = [3,3].
    Experts: I0 = {0}, I1 = {2}. Routing: q0 -> 0, q1 = 0 (tie) -> 0, q2 -> 1, q3 -> 0.
    q0's logits over [q~0, q~1, K0] are [sqrt2, 0, 2 ln2] with values [V~0, V~1, V0]."""
    r2, l2 = math.sqrt(2.0), math.log(2.0)
    Q = np.array([[2, 0], [0, 0], [0, 2], [0, 0]], dtype=np.float64)
    K = r2 * np.array([[l2, 0], [0, 0], [0, l2], [0, 0]])
    V = np.array([[5, 0], [0, 5], [0, 0], [10, 10]], dtype=np.float64)
    r = oracle.forward(Q, K, V, 1, 4, 1, 2, 1, 1)
    np.testing.assert_allclose(r["Qt"], [[1, 0], [0, 1]], atol=1e-15)
    np.testing.assert_allclose(r["Vt"], [[4, 3], [3, 3]], atol=1e-13)
    assert r["I"].tolist() == [[0], [2]]
    assert r["E"].ravel().tolist() == [0, 0, 1, 0]
    e = math.exp(r2)
    want = np.array([
        (e * np.array([4, 3]) + np.array([3, 3]) + 4 * np.array([5, 0])) / (e + 5),
        [4, 2],
        (np.array([4, 3]) + e * np.array([3, 3])) / (5 + e),
        [4, 2],
    ])
    np.testing.assert_allclose(r["O"], want, rtol=1e-13, atol=1e-13)


def _full_attention_with_bias(Q, keys, vals, bias):
    return F.scaled_dot_product_attention(
        torch.from_numpy(Q)[None, None], torch.from_numpy(keys)[None, None],
        torch.from_numpy(vals)[None, None], attn_mask=torch.from_numpy(bias)[None, None])[0, 0].numpy()


def test_k_equals_n_s_equals_1_is_full_attention_over_landmarks_and_keys():
    N, d, m = 96, 16, 8
    Q, K, V = rand((N, d), 20), rand((N, d), 21), rand((N, d), 22)
    r = oracle.forward(Q, K, V, 1, N, 1, m, N, 1)
    keys, vals = np.concatenate([r["Qt"], K]), np.concatenate([r["Vt"], V])
    ref = _full_attention_with_bias(Q, keys, vals, np.zeros((N, m + N)))
    np.testing.assert_allclose(r["O"], ref, rtol=1e-11, atol=1e-12)


def test_k_equals_n_s_equals_m_adds_ln_m_to_key_logits():
    # every token sits in all m experts, so each key appears m times
    N, d, m = 64, 8, 4
    Q, K, V = rand((N, d), 23), rand((N, d), 24), rand((N, d), 25)
    r = oracle.forward(Q, K, V, 1, N, 1, m, N, m)
    keys, vals = np.concatenate([r["Qt"], K]), np.concatenate([r["Vt"], V])
    bias = np.concatenate([np.zeros((N, m)), np.full((N, N), math.log(m))], axis=1)
    np.testing.assert_allclose(r["O"], _full_attention_with_bias(Q, keys, vals, bias), rtol=1e-11, atol=1e-12)


def test_output_linear_in_v_and_shift_equivariant():
    N, d, m, k, s = 80, 8, 8, 10, 2
    Q, K = rand((N, d), 26), rand((N, d), 27)
    V1, V2 = rand((N, d), 28), rand((N, d), 29)
    f = lambda V: oracle.forward(Q, K, V, 1, N, 1, m, k, s)["O"]
    np.testing.assert_allclose(f(2.0 * V1 - 3.0 * V2), 2.0 * f(V1) - 3.0 * f(V2), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(f(V1 + 0.75), f(V1) + 0.75, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f(np.ones((N, d))), 1.0, atol=1e-14)   # weights sum to 1


def test_joint_permutation_of_keys_and_values():
    N, d, m, k, s = 60, 8, 6, 7, 2
    Q, K, V = rand((N, d), 30), rand((N, d), 31), rand((N, d), 32)
    pi = np.random.default_rng(33).permutation(N)
    a = oracle.forward(Q, K, V, 1, N, 1, m, k, s)
    b = oracle.forward(Q, K[pi], V[pi], 1, N, 1, m, k, s)
    # token n of the permuted input is token pi[n] of the original
    np.testing.assert_array_equal(np.sort(pi[b["I"]], axis=1), a["I"])
    np.testing.assert_array_equal(a["E"], b["E"])
    np.testing.assert_allclose(b["O"], a["O"], rtol=1e-12, atol=1e-13)


def test_single_landmark_is_mean_query():
    N, d = 50, 4
    Q, K, V = rand((N, d), 34), rand((N, d), 35), rand((N, d), 36)
    r = oracle.forward(Q, K, V, 1, N, 1, 1, 5, 1)
    np.testing.assert_allclose(r["Qt"][0], Q.mean(axis=0), rtol=1e-14)
    assert (r["E"] == 0).all()


def test_duplicates_across_experts_are_kept():
    # a key shared by both routed experts counts twice: compare with an explicit list
    N, d, m, k, s = 32, 4, 2, 32, 2
    Q, K, V = rand((N, d), 37), rand((N, d), 38), rand((N, d), 39)
    r = oracle.forward(Q, K, V, 1, N, 1, m, k, s)
    keys = np.concatenate([r["Qt"], K, K])
    vals = np.concatenate([r["Vt"], V, V])
    np.testing.assert_allclose(r["O"], _full_attention_with_bias(Q, keys, vals, np.zeros((N, m + 2 * N))),
                               rtol=1e-11, atol=1e-12)


def test_sampled_queries_match_full_output():
    w = synth.WORKLOADS["tiny"]
    Q, K, V = (x[0, 0] for x in synth.make_inputs(w))
    full = oracle.forward(Q, K, V, w.grid_h, w.grid_w, w.pool_h, w.pool_w, w.k, w.s)
    qs = [0, 5, 1023, 512]
    part = oracle.forward(Q, K, V, w.grid_h, w.grid_w, w.pool_h, w.pool_w, w.k, w.s, queries=qs)
    np.testing.assert_array_equal(part["O"], full["O"][qs])
    np.testing.assert_array_equal(part["E"][qs], full["E"][qs])


# ---------------------------------------------------------------- validity rule

def test_validity_rule():
    S = np.array([[5.0, 4.0, 3.0, 3.0 * (1 - 1e-8), 1.0]])
    assert oracle.valid_topk_sets(S, np.array([[0, 1, 2]]), 3)[0]
    assert oracle.valid_topk_sets(S, np.array([[0, 1, 3]]), 3)[0]       # near-tie swap allowed
    assert not oracle.valid_topk_sets(S, np.array([[0, 1, 4]]), 3)[0]   # clear loser
    assert not oracle.valid_topk_sets(S, np.array([[0, 2, 3]]), 3)[0]   # drops a clear winner
    assert not oracle.valid_topk_sets(S, np.array([[0, 1, 1]]), 3)[0]   # duplicate


# ---------------------------------------------------------------- margins
# The margin decides which rows must equal the oracle's set exactly (relative
# gap between the k-th and (k+1)-th largest score at least 1e-6). Hand-worked
# values: the row's scores sorted by hand, the gap divided by |k-th score|.

def test_topk_margins_hand_worked():
    S = np.array([
        [5.0, 3.0, 3.000001, 1.0],   # sorted 5, 3.000001, 3, 1: k = 2 -> 1e-6 / 3.000001
        [1.0, 2.0, 0.0, 1.0],        # sorted 2, 1, 1, 0: exact tie at the cut, 0
        [-1.0, -4.0, -2.0, -8.0],    # negative k-th score: (-2 - (-4)) / |-2| = 1
        [0.0, 7.0, -1.0, -3.0],      # sorted 7, 0, -1, -3: k-th score 0, gap 1 / 1e-300 (finite)
    ])
    got = oracle.topk_margins(S, 2)
    assert got[0] == pytest.approx(1e-6 / 3.000001, rel=1e-9)
    assert got[1] == 0.0
    assert got[2] == 1.0
    assert got[3] == pytest.approx(1.0 / 1e-300, rel=1e-12)
    # k = 1 uses the largest and second largest; k = 3 the third and fourth
    np.testing.assert_allclose(oracle.topk_margins(S[:1], 1), [(5.0 - 3.000001) / 5.0], rtol=1e-14)
    np.testing.assert_allclose(oracle.topk_margins(S[:1], 3), [(3.0 - 1.0) / 3.0], rtol=1e-14)


def test_topk_margins_k_equals_n_is_inf():
    S = rand((3, 5), 11)
    assert np.isinf(oracle.topk_margins(S, 5)).all()
    assert np.isfinite(oracle.topk_margins(S, 4)).all()


def test_route_margins_hand_worked():
    # router row q . q~_i = [0.5, 2.0, 1.0, 1.5]: s = 2 -> (1.5 - 1.0) / 1.5; s = 1 -> (2 - 1.5) / 2
    R = np.array([[0.5, 2.0, 1.0, 1.5], [1.0, 1.0, 1.0, 1.0]])
    np.testing.assert_allclose(oracle.route_margins(R, 2), [1.0 / 3.0, 0.0], rtol=1e-14)
    np.testing.assert_allclose(oracle.route_margins(R, 1), [0.25, 0.0], rtol=1e-14)
    assert np.isinf(oracle.route_margins(R, 4)).all()


def test_margins_brute_force_random_rows():
    # pure-Python sort of each row, gap taken by the definition
    S = rand((20, 13), 12)
    S[3, 5] = S[3, 7]   # one exact tie
    for k in (1, 4, 12):
        got = oracle.topk_margins(S, k)
        for i, row in enumerate(S.tolist()):
            srt = sorted(row, reverse=True)
            want = (srt[k - 1] - srt[k]) / max(abs(srt[k - 1]), 1e-300)
            assert got[i] == pytest.approx(want, rel=1e-13, abs=0.0)


def test_margins_agree_with_validity_rule():
    # a row with margin >= 1e-6 admits exactly one valid set (the oracle's); a row
    # below it admits a swap across the cut
    S = np.array([[4.0, 3.0, 3.0 * (1 - 1e-7), 1.0], [4.0, 3.0, 2.0, 1.0]])
    marg = oracle.topk_margins(S, 2)
    assert marg[0] < 1e-6 <= marg[1]
    assert oracle.valid_topk_sets(S[:1], np.array([[0, 2]]), 2)[0]
    assert not oracle.valid_topk_sets(S[1:], np.array([[0, 2]]), 2)[0]


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_sliceable():
    w = synth.WORKLOADS["vit_b"]
    a = synth.make_inputs(w, slices=[(3, 5)])
    b = synth.make_inputs(w, slices=[(3, 5)])
    c = synth.make_inputs(w, slices=[(3, 6)])
    for x, y, z in zip(a, b, c):
        assert x.dtype == np.uint16 and x.shape == (1, 3136, 64)
        np.testing.assert_array_equal(x, y)
        assert (x != z).any()


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 4 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -7], np.float32))


def test_needles_scale_keys_only():
    w = synth.WORKLOADS["long"].with_(N=4096)
    Q, K, V = synth.draw_slice(w, 0, 0)
    w0 = w.with_(needle_frac=0.0)
    Q0, K0, V0 = synth.draw_slice(w0, 0, 0)
    np.testing.assert_array_equal(Q, Q0)
    np.testing.assert_array_equal(V, V0)
    changed = np.nonzero((K != K0).any(axis=1))[0]
    assert len(changed) == round(0.01 * 4096)
    np.testing.assert_array_equal(K[changed], 4 * K0[changed])


# Standard attention over all keys (the baseline the pages compare MiTA with;
# the GPU comparator kernel is checked against oracle.full_attention).
@pytest.mark.parametrize("N,d", [(1, 8), (37, 16), (300, 64)])
def test_full_attention_matches_torch_sdpa(N, d):
    Q, K, V = rand((N, d), 30), rand((N, d), 31), rand((N, d), 32)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x)[None, None] for x in (Q, K, V)))[0, 0].numpy()
    np.testing.assert_allclose(oracle.full_attention(Q, K, V), ref, rtol=1e-12, atol=1e-13)


def test_full_attention_brute_force():
    N, d = 5, 3
    Q, K, V = rand((N, d), 33), rand((N, d), 34), rand((N, d), 35)
    out = oracle.full_attention(Q, K, V)
    for i in range(N):
        w = [math.exp(sum(Q[i, c] * K[j, c] for c in range(d)) / math.sqrt(d)) for j in range(N)]
        for c in range(d):
            assert abs(out[i, c] - sum(w[j] * V[j, c] for j in range(N)) / sum(w)) < 1e-13


def test_full_attention_closed_forms():
    N, d = 50, 8
    Q, V = rand((N, d), 36), rand((N, d), 37)
    # identical keys: uniform weights, every row is the mean of V
    K = np.tile(rand((1, d), 38), (N, 1))
    np.testing.assert_allclose(oracle.full_attention(Q, K, V), np.tile(V.mean(axis=0), (N, 1)), rtol=1e-13, atol=1e-14)
    # one key far above the rest for every query: the output is its value row
    K = np.zeros((N, d))
    K[7, 0] = 1e3
    Qp = np.abs(Q) + 1.0
    np.testing.assert_allclose(oracle.full_attention(Qp, K, V), np.tile(V[7], (N, 1)), rtol=0, atol=1e-12)
