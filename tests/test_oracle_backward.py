"""Pins of the fp64 oracle's backward pass (gradients of sum(dO * O) with the
expert sets and the routing held fixed) against things other than itself:
central finite differences of the pinned forward oracle, torch autograd in fp64
through a forward built from torch's own pooling and attention routines, a
closed-form invariant, linearity, and planted slips that each fail. CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import mita_oracle as mo

torch.set_default_dtype(torch.float64)


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def problem(N=12, d=4, gh=1, gw=None, ph=1, pw=3, k=5, s=2, seed=0):
    gw = N if gw is None else gw
    Q, K, V = rand((N, d), seed), rand((N, d), seed + 1), rand((N, d), seed + 2)
    dO = rand((N, d), seed + 3)
    r = oracle.forward(Q, K, V, gh, gw, ph, pw, k, s)
    return dict(Q=Q, K=K, V=V, dO=dO, I=r["I"], E=r["E"], grid=(gh, gw), pool=(ph, pw))


def loss(Q, K, V, p):
    """sum(dO * O) through the forward oracle, expert sets and routing held fixed."""
    Qt = oracle.pool(Q, *p["grid"], *p["pool"])
    Vt = oracle.shared_expert(Qt, K, V)
    return float((p["dO"] * oracle.attend(Q, K, V, Qt, Vt, p["I"], p["E"])).sum())


def finite_difference_grads(p, h=1e-6):
    out = {}
    for name in ("Q", "K", "V"):
        g = np.zeros_like(p[name])
        for idx in np.ndindex(*g.shape):
            args = {n: p[n].copy() for n in ("Q", "K", "V")}
            args[name][idx] += h
            up = loss(args["Q"], args["K"], args["V"], p)
            args[name][idx] -= 2 * h
            dn = loss(args["Q"], args["K"], args["V"], p)
            g[idx] = (up - dn) / (2 * h)
        out["d" + name] = g
    return out


def oracle_grads(p, dO=None):
    return oracle.backward(p["Q"], p["K"], p["V"], *p["grid"], *p["pool"], p["I"], p["E"],
                           p["dO"] if dO is None else dO)


CASES = [
    dict(),                                              # 1D, s = 2 (duplicates across a query's experts)
    dict(N=20, d=3, gh=4, gw=5, ph=2, pw=2, k=6, s=3),   # 2D grid, overlapping experts
    dict(N=10, d=4, pw=3, k=10, s=3),                    # k = N, s = m: every token in every expert
    dict(N=9, d=2, pw=4, k=3, s=1),                      # windows overlap (9 tokens to 4 cells)
]


@pytest.mark.parametrize("kw", CASES, ids=["1d_s2", "2d_s3", "kN_sm", "overlap_s1"])
def test_backward_matches_finite_differences(kw):
    p = problem(**kw)
    got = oracle_grads(p)
    fd = finite_difference_grads(p)
    for n in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(got[n], fd[n], rtol=1e-6, atol=1e-7, err_msg=n)


def torch_forward(Q, K, V, p):
    """The forward built from torch routines: adaptive average pooling, SDPA for the
    shared expert, and an explicit gather-and-concatenate final attention with the
    fixed index sets; differentiated by autograd."""
    gh, gw = p["grid"]
    ph, pw = p["pool"]
    N, d = Q.shape
    img = Q.T.reshape(1, d, gh, gw)
    Qt = F.adaptive_avg_pool2d(img, (ph, pw)).reshape(d, ph * pw).T
    Vt = F.scaled_dot_product_attention(Qt[None, None], K[None, None], V[None, None])[0, 0]
    I = torch.as_tensor(np.asarray(p["I"]), dtype=torch.long)
    E = torch.as_tensor(np.asarray(p["E"]), dtype=torch.long)
    outs = []
    for q in range(N):
        toks = I[E[q]].reshape(-1)
        Ks = torch.cat([Qt, K[toks]], 0)
        Vs = torch.cat([Vt, V[toks]], 0)
        w = torch.softmax(Ks @ Q[q] / math.sqrt(d), 0)
        outs.append(w @ Vs)
    return torch.stack(outs)


@pytest.mark.parametrize("kw", CASES + [dict(N=64, d=8, gh=8, gw=8, ph=4, pw=2, k=16, s=3, seed=5)],
                         ids=["1d_s2", "2d_s3", "kN_sm", "overlap_s1", "larger_2d"])
def test_backward_matches_torch_autograd(kw):
    p = problem(**kw)
    Q, K, V = (torch.tensor(p[n], requires_grad=True) for n in ("Q", "K", "V"))
    O = torch_forward(Q, K, V, p)
    # the torch forward is the oracle's forward (pinned elsewhere) ...
    np.testing.assert_allclose(O.detach().numpy(), oracle.attend(
        p["Q"], p["K"], p["V"], oracle.pool(p["Q"], *p["grid"], *p["pool"]),
        oracle.shared_expert(oracle.pool(p["Q"], *p["grid"], *p["pool"]), p["K"], p["V"]), p["I"], p["E"]),
        rtol=1e-12, atol=1e-13)
    # ... and autograd differentiates it independently of the oracle's chain rule
    (O * torch.from_numpy(p["dO"])).sum().backward()
    got = oracle_grads(p)
    for n, t in (("dQ", Q), ("dK", K), ("dV", V)):
        np.testing.assert_allclose(got[n], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)


def test_value_gradient_mass_is_sum_of_output_gradients():
    # every query's weights sum to 1 and so does every shared-expert row, so the
    # value gradients of all tokens add up to the sum of the output gradients
    for kw in CASES:
        p = problem(**kw)
        got = oracle_grads(p)
        np.testing.assert_allclose(got["dV"].sum(axis=0), p["dO"].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_backward_linear_in_output_gradient():
    p = problem(N=16, d=4, pw=4, k=6, s=2, seed=7)
    a, b = rand(p["dO"].shape, 8), rand(p["dO"].shape, 9)
    ga, gb, gab = oracle_grads(p, a), oracle_grads(p, b), oracle_grads(p, a + 2.0 * b)
    for n in ("dQ", "dK", "dV"):
        np.testing.assert_allclose(gab[n], ga[n] + 2.0 * gb[n], rtol=1e-11, atol=1e-12)
    z = oracle_grads(p, np.zeros_like(a))
    assert all(not np.abs(z[n]).max() for n in ("dQ", "dK", "dV"))


def test_pool_matrix_reproduces_pooling():
    for gh, gw, ph, pw in ((1, 10, 1, 4), (4, 5, 2, 3), (6, 6, 6, 6)):
        Q = rand((gh * gw, 3), gh + gw)
        np.testing.assert_allclose(oracle.pool_matrix(gh * gw, gh, gw, ph, pw) @ Q, oracle.pool(Q, gh, gw, ph, pw),
                                   rtol=1e-14, atol=1e-14)
