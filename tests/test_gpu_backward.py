"""GPU parity of the backward pass (bf16): mita_backward through the C ABI
against the fp64 oracle's backward, evaluated with the GPU's own (validated)
expert sets and routing held fixed. Tolerance: every contraction takes bf16
operands (unit roundoff 2^-9), dS = P (dP - D) loses relative accuracy where dP
and D nearly cancel, and the recompute takes the bf16 part of Q~; the bar is a
max-abs error of 2e-2 x the largest magnitude of each reference gradient, per
slice. Gradients are also checked bit-identical across two calls."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import say, slice_f64, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
TOL_GRAD = 2e-2


def small(name, **kw):
    return W["tiny"].with_(name=name, dtype="bf16", **kw)


CASES = [
    # s = 3: partials + combine forward, routed query tiles of 64 rows
    small("bwd_ragged_s3", B=2, H=2, N=1000, grid_w=1000, pool_w=10, k=37, s=3),
    # d = 128, routed tiles of 128 rows (mean bucket >= 256)
    small("bwd_d128_s5", B=1, H=2, N=2048, d=128, grid_w=2048, pool_w=8, k=64, s=5, ncl=8),
    # 2D grid with overlapping pooling windows; s = 1 one-pass forward
    small("bwd_grid2d_overlap", B=1, H=2, N=30 * 33, grid_h=30, grid_w=33, pool_h=4, pool_w=5, k=50, s=1),
    # m > 64 (several landmark blocks), k > 64 (several key blocks per expert)
    small("bwd_m100_k130", B=1, H=1, N=5000, grid_w=5000, pool_w=100, k=130, s=2),
    # k = N, s = m: every token in every expert (long inverse lists)
    small("bwd_kN_sm", B=1, H=1, N=256, grid_w=256, pool_w=4, k=256, s=4),
    # needle keys: tokens held by many experts
    small("bwd_needles_d128", B=1, H=1, N=4096, d=128, grid_w=4096, pool_w=32, k=128, s=2, needle_frac=0.01),
]


def run_gpu(w, lib, seed=7):
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    call.pool(Qd)
    call.landmark(Kd, Vd)
    I = call.topk(Kd, want=True)
    E = call.route(Qd, want=True)
    O = call.output(Qd, Kd, Vd)
    rng = np.random.default_rng(seed)
    dO = synth.f32_to_bf16_bits(rng.standard_normal(Q.shape, dtype=np.float32)).reshape(Q.shape)
    dOd = to_device(dO, "bf16")
    g1 = [t.clone() for t in call.backward(Qd, Kd, Vd, O, dOd)]
    g2 = call.backward(Qd, Kd, Vd, O, dOd)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "backward is not deterministic"
    return Q, K, V, dO, I.cpu().numpy(), E.cpu().numpy(), [g.cpu().numpy().astype(np.float64) for g in g1]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward_matches_oracle(w, lib):
    say(f"[backward] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} k={w.k} s={w.s}")
    Q, K, V, dO, I, E, grads = run_gpu(w, lib)
    for z in range(w.slices):
        q64, k64, v64, do64 = (slice_f64(x, "bf16", z) for x in (Q, K, V, dO))
        Iz = I.reshape(-1, w.m, w.k)[z].astype(np.int64)
        Ez = E.reshape(-1, w.N, w.s)[z].astype(np.int64)
        ref = oracle.backward(q64, k64, v64, w.grid_h, w.grid_w, w.pool_h, w.pool_w, Iz, Ez, do64)
        errs = {}
        for name, g in zip(("dQ", "dK", "dV"), grads):
            gz = g.reshape(-1, w.N, w.d)[z]
            scale = np.abs(ref[name]).max()
            errs[name] = np.abs(gz - ref[name]).max() / scale
            assert errs[name] <= TOL_GRAD, f"slice {z} {name}: max error {errs[name]:.3g} x max|ref|"
        say(f"  slice {z}: relative max errors " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))


def test_backward_full_size_invariant(lib):
    """The long workload whole (B=2, H=16, N=65536, d=128, m=256, k=256, s=2): every
    query's weights and every shared-expert row sum to 1, so per slice the value
    gradients add up to the sum of the output gradients; all gradients finite; a
    second call is bit-identical (the forward fills its buckets in atomic order
    from many workgroups at this size; the backward must not depend on it)."""
    w = W["long"]
    say("[backward-full] long: forward + backward")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    O = call.forward(Qd, Kd, Vd)
    dOd = (torch.randn(Qd.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(3))).to(torch.bfloat16)
    dQ, dK, dV = (t.clone() for t in call.backward(Qd, Kd, Vd, O, dOd))
    O2 = call.forward(Qd, Kd, Vd)   # buckets refilled
    g2 = call.backward(Qd, Kd, Vd, O2, dOd)
    torch.cuda.synchronize()
    assert torch.equal(O, O2)
    for name, a, b in zip(("dQ", "dK", "dV"), (dQ, dK, dV), g2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} differs between two calls"
    for g in (dQ, dK, dV):
        assert torch.isfinite(g).all()
    lhs = dV.double().sum(dim=2)
    rhs = dOd.double().sum(dim=2)
    err = (lhs - rhs).abs().max().item() / rhs.abs().max().item()
    say(f"  value-gradient mass: max relative error {err:.2e}")
    assert err <= TOL_GRAD
