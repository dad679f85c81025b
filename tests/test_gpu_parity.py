"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded input bits. Index sets must be exact except on near-ties (relative
k-th/(k+1)-th gap below 1e-6); outputs within max-abs 2e-2 (bf16) or 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

import synth
from helpers import TOL_OUT, check_slice, run_gpu_steps, say, slice_f64, to_device, out_to_f64

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def small(name, **kw):
    return W["tiny"].with_(name=name, **kw)


# Several tiles and ragged tails: N not a multiple of 64 (or of 4), 2D grids with
# overlapping windows, both head sizes, both dtypes, every router path (fast
# lists of 4, 6 and 8 entries, and the exact kernel for s > 6).
SMALL = [
    W["tiny"],
    small("ragged_bf16", B=2, H=2, N=1000, grid_w=1000, pool_w=10, k=37, s=3, dtype="bf16"),
    small("ragged_f32_d128", B=1, H=3, N=777, d=128, grid_w=777, pool_w=13, k=100, s=2),
    small("grid2d_overlap", B=1, H=2, N=30 * 33, grid_h=30, grid_w=33, pool_h=4, pool_w=5, k=50, s=1, dtype="bf16"),
    small("d128_s5", B=1, H=2, N=2048, d=128, grid_w=2048, pool_w=32, k=64, s=5, dtype="bf16", ncl=8),
    small("exact_router_s7", B=1, H=1, N=1536, grid_w=1536, pool_w=24, k=40, s=7, dtype="bf16"),
    small("multi_segment", B=1, H=1, N=20000, grid_w=20000, pool_w=40, k=300, s=2, dtype="bf16", needle_frac=0.01),
    small("odd_n", B=1, H=1, N=1001, grid_w=1001, pool_w=7, k=1001, s=7, dtype="bf16"),
    # s = 1 with one key block per expert (k, m <= 64): the one-pass output kernel
    small("one_block_f32_d128", B=2, H=1, N=700, d=128, grid_w=700, pool_w=50, k=33, s=1),
    small("one_block_bf16_d128", B=1, H=3, N=4096, d=128, grid_w=4096, pool_w=64, k=64, s=1, dtype="bf16"),
    # fp32 over several key chunks; several landmark tiles per slice on a 2D grid
    small("chunked_f32", B=1, H=2, N=5000, grid_w=5000, pool_w=20, k=80, s=2),
    small("tiles_2d_bf16", B=1, H=2, N=64 * 64, grid_h=64, grid_w=64, pool_h=10, pool_w=10, k=64, s=2,
          dtype="bf16"),
    # s = 1 with k > 64 and d = 128: the general kernel with the landmark part fused
    small("fused_bf16_d128", B=1, H=2, N=3000, d=128, grid_w=3000, pool_w=30, k=100, s=1, dtype="bf16"),
    # m > 64 with s = 1: router lists of order keys carrying the landmark id, and the
    # general kernel streaming the landmark blocks (not resident)
    small("landmarks100_s1", B=1, H=2, N=5000, grid_w=5000, pool_w=100, k=64, s=1, dtype="bf16"),
    # fp32 with m > 64 (the router's fp32 MFMA path with key lists)
    small("f32_m80", B=1, H=2, N=4000, grid_w=4000, pool_w=80, k=50, s=2),
    # fewer group maxima per row than k: no threshold, all N scores are candidates of
    # the select kernel (N <= 4096) ...
    small("k1100_all_candidates", B=1, H=1, N=3000, grid_w=3000, pool_w=8, k=1100, s=1, dtype="bf16"),
    # ... or, past its capacity, every row is selected from fp64 scores of the whole row
    small("k1100_fallback", B=1, H=2, N=5000, grid_w=5000, pool_w=8, k=1100, s=1, dtype="bf16"),
    # more than 4096 group maxima per row (groups of 16 since k > N / 256): no candidate
    # threshold, so every row overflows its lists and goes to the fp64 fallback
    small("no_threshold", B=1, H=1, N=70000, grid_w=70000, pool_w=8, k=300, s=1, dtype="bf16"),
]

# bf16, m > 64 and at least 4 k blocks of 64 keys, with k < 64: expert sets came out
# all 0 on the first and a second call faulted; the library refuses bf16 with m > 64,
# k < 64 and N >= 256 k until the cause is found (test_abi checks the refusal)
SMALL_K_BF16 = [
    small("candidate_skip_d128", B=1, H=2, N=12000, d=128, grid_w=12000, pool_w=150, k=32, s=2, dtype="bf16",
          needle_frac=0.01),
    small("candidate_skip_d64", B=1, H=1, N=9001, grid_w=9001, pool_w=96, k=20, s=2, dtype="bf16"),
]


# The inference-time (m, k, s) settings that bench.py --sweep times, on two
# slices of the ViT-B-like inputs.
SWEEP = [w.with_(B=1, H=2) for w in synth.sweep_workloads("vit_b")]


@pytest.mark.parametrize("w", SWEEP, ids=lambda w: w.name)
def test_sweep_settings(w, lib):
    say(f"[sweep] {w.name}")
    Q, K, V = synth.make_inputs(w)
    gpu = run_gpu_steps(w, Q, K, V, lib, want_s=False)
    for z in range(w.slices):
        st = check_slice(w, Q, K, V, gpu, z, check_s=False)
        say(f"  slice {z}: {st}")


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_workloads_all_slices(w, lib):
    say(f"[parity] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} k={w.k} s={w.s} {w.dtype}")
    Q, K, V = synth.make_inputs(w)
    gpu = run_gpu_steps(w, Q, K, V, lib)
    for z in range(w.slices):
        st = check_slice(w, Q, K, V, gpu, z)
        say(f"  slice {z}: {st}")


@pytest.mark.skip(reason="bf16 with m > 64, k < 64 and N >= 256 k gave all-0 expert sets and a memory fault; refused by the library until the cause is found")
@pytest.mark.parametrize("w", SMALL_K_BF16, ids=lambda w: w.name)
def test_small_k_bf16_many_landmarks(w, lib):
    say(f"[parity] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} k={w.k} s={w.s} {w.dtype}")
    Q, K, V = synth.make_inputs(w)
    gpu = run_gpu_steps(w, Q, K, V, lib)
    for z in range(w.slices):
        st = check_slice(w, Q, K, V, gpu, z)
        say(f"  slice {z}: {st}")


def test_forward_equals_steps_and_is_deterministic(lib):
    w = SMALL[1]
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, pool=(w.pool_h, w.pool_w))
    a = call.forward(Qd, Kd, Vd).clone()
    b = call.forward(Qd, Kd, Vd).clone()
    call.pool(Qd)
    call.landmark(Kd, Vd)
    call.topk(Kd)
    call.route(Qd)
    c = call.output(Qd, Kd, Vd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_full_attention_reduction(lib):
    # k = N: every expert holds every token; s = m adds ln m to every key logit
    import oracle
    for s in (1, 4):
        w = small("kN", N=256, grid_w=256, pool_w=4, k=256, s=s)
        Q, K, V = synth.make_inputs(w)
        gpu = run_gpu_steps(w, Q, K, V, lib)
        check_slice(w, Q, K, V, gpu, 0)
        assert (np.sort(gpu["I"][0, 0], axis=1) == np.arange(256)).all()


def test_degenerate_ties(lib):
    # all-zero keys: every score ties, so experts are the k lowest token ids;
    # all-zero queries: every router score ties, so queries go to experts 0..s-1
    w = small("ties", N=4096, grid_w=4096, pool_w=16, k=100, s=2, dtype="bf16")
    Q, K, V = synth.make_inputs(w)
    K[:] = 0
    Q[..., :2048, :] = 0
    gpu = run_gpu_steps(w, Q, K, V, lib)
    assert (gpu["I"][0, 0] == np.arange(100)[None, :]).all()
    assert (gpu["E"][0, 0, :2048] == np.array([0, 1])[None, :]).all()
    check_slice(w, Q, K, V, gpu, 0)


def test_partials_scale_with_v(lib):
    """With s > 1 each slot's partial output is stored relative to its own largest
    magnitude (fp16 for bf16 inputs): values far beyond fp16's range pass through,
    scaling V by a power of two scales the output by exactly that power (bit for
    bit: every rounding on the way scales with it), and V = 0 gives exactly 0."""
    for dt in ("bf16", "f32"):
        w = small(f"v_scale_{dt}", B=1, H=2, N=3000, grid_w=3000, pool_w=30, k=70, s=3, dtype=dt)
        say(f"[v-scale] {w.name}")
        Q, K, V = synth.make_inputs(w)
        Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
        call = lib.Mita.create(Qd, w.m, w.k, w.s, pool=(w.pool_h, w.pool_w))
        a = call.forward(Qd, Kd, Vd).clone()
        b = call.forward(Qd, Kd, Vd * 2.0 ** 20).clone()
        c = call.forward(Qd, Kd, torch.zeros_like(Vd))
        torch.cuda.synchronize()
        assert b.float().abs().max().item() > 65504.0
        assert torch.equal(a.float() * 2.0 ** 20, b.float())
        assert not c.float().abs().max().item()


def test_single_landmark_and_identity_pool(lib):
    for pw, k, s in ((1, 20, 1), (128, 5, 3)):
        w = small(f"pool{pw}", N=128, grid_w=128, pool_w=pw, k=k, s=s, dtype="bf16")
        Q, K, V = synth.make_inputs(w)
        gpu = run_gpu_steps(w, Q, K, V, lib)
        check_slice(w, Q, K, V, gpu, 0)


def test_invalid_arguments_raise(lib):
    w = W["tiny"]
    Q = torch.zeros((1, 1, 1024, 64), device="cuda")
    with pytest.raises(ValueError):
        lib.Mita.create(Q, 16, 2000, 1)           # k > N
    with pytest.raises(ValueError):
        lib.Mita.create(Q, 16, 64, 17)            # s > m
    with pytest.raises(ValueError):
        lib.Mita.create(torch.zeros((1, 1, 64, 96), device="cuda"), 4, 8, 1)   # d = 96 unsupported


FULL = ["vit_b", "seg", "long", "very_long"]
# slices z = b H + h checked at full size: two per workload, different heads (and
# batch entries where there is more than one)
FULL_SLICES = {"vit_b": [0, 383], "seg": [0, 95], "long": [3, 28], "very_long": [2, 6]}
FULL_QUERIES = 2048   # random queries per slice whose output is checked


def full_size_queries(E_z: np.ndarray, N: int, rng) -> np.ndarray:
    """Queries whose output is checked: a random sample, plus the highest query
    routed to each expert (the tail of every expert's bucket, so partially filled
    last tiles are covered)."""
    rand = rng.choice(N, size=min(N, FULL_QUERIES), replace=False)
    flat_e = E_z.reshape(-1)
    flat_q = np.repeat(np.arange(N), E_z.shape[1])
    last = np.full(int(flat_e.max()) + 1, -1, dtype=np.int64)
    np.maximum.at(last, flat_e, flat_q)
    return np.union1d(rand, last[last >= 0])


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name, lib):
    """Whole workload through mita_forward (the launch configuration the benchmark
    times), checked on sampled slices and queries."""
    w = W[name]
    say(f"[parity-full] {name}: generating")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    say(f"[parity-full] {name}: forward")
    O = call.forward(Qd, Kd, Vd)
    torch.cuda.synchronize()
    say(f"[parity-full] {name}: steps")
    Qt = call.pool(Qd, want=True)
    Vt, _ = call.landmark(Kd, Vd, want_vt=True)
    I = call.topk(Kd, want=True)
    E = call.route(Qd, want=True)
    O2 = call.output(Qd, Kd, Vd)
    torch.cuda.synchronize()
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16))
    gpu = {"Qt": Qt.cpu().numpy(), "Vt": Vt.cpu().numpy().astype(np.float64), "I": I.cpu().numpy(),
           "E": E.cpu().numpy(), "O": out_to_f64(O)}
    del Qd, Kd, Vd, call
    rng = np.random.default_rng(1)
    for z in FULL_SLICES[name]:
        queries = full_size_queries(gpu["E"].reshape(-1, w.N, w.s)[z], w.N, rng)
        say(f"[parity-full] {name}: oracle on slice {z} (routing of all {w.N} queries, output of "
            f"{len(queries)} + 256 nearest a routing tie)")
        st = check_slice(w, Q, K, V, gpu, z, queries=queries, check_s=False, route_all=True, near_margin=256)
        say(f"  slice {z}: {st}")


def test_forward_on_a_side_stream_and_in_a_graph(lib):
    """mita_forward runs on the stream it is given (here a non-default torch
    stream) and can be captured into a HIP graph; every replay, with eager work
    between replays, must match the eager output bit for bit."""
    w = SMALL[1]
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, pool=(w.pool_h, w.pool_w))
    ref = call.forward(Qd, Kd, Vd).clone()           # eager, default stream (also creates the side stream)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    out = torch.empty_like(Qd)
    with torch.cuda.stream(st):
        call.forward(Qd, Kd, Vd, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))

    g = torch.cuda.CUDAGraph()
    gout = torch.empty_like(Qd)
    with torch.cuda.graph(g, stream=st):
        call.forward(Qd, Kd, Vd, gout)
    torch.cuda.synchronize()
    for rep in range(4):
        gout.zero_()
        eager = call.forward(Qd, Kd, Vd)             # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gout.view(torch.int16), ref.view(torch.int16)), f"replay {rep} differs"
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))


# The full-attention comparator (standard softmax attention over all N keys):
# ragged N, both head sizes and dtypes, several XCD groups, a single key.
DENSE = [
    small("dense_bf16", B=1, H=2, N=1000, grid_w=1000, pool_w=10, dtype="bf16"),
    small("dense_f32_d128", B=2, H=1, N=777, d=128, grid_w=777, pool_w=7),
    small("dense_bf16_d128", B=1, H=1, N=4100, d=128, grid_w=4100, pool_w=41, dtype="bf16"),
    small("dense_f32_many_tiles", B=3, H=7, N=300, grid_w=300, pool_w=3),
    small("dense_one_key", B=1, H=3, N=1, grid_w=1, pool_w=1, k=1, s=1, dtype="bf16"),
]


@pytest.mark.parametrize("w", DENSE, ids=lambda w: w.name)
def test_dense_attention(w, lib):
    import oracle
    say(f"[dense] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    O = lib.dense_attention(Qd, Kd, Vd)
    torch.cuda.synchronize()
    O = out_to_f64(O).reshape(-1, w.N, w.d)
    for z in range(w.slices):
        ref = oracle.full_attention(*(slice_f64(x, w.dtype, z) for x in (Q, K, V)))
        err = np.abs(O[z] - ref).max()
        assert err <= TOL_OUT[w.dtype], f"slice {z}: max abs error {err:.3g}"


@pytest.mark.parametrize("name", ["vit_b", "seg", "long"])
def test_dense_attention_full_size_sampled(name, lib):
    """The comparator on whole workloads (the launches bench.py --dense times),
    checked on sampled queries of two slices (each query row is independent)."""
    import oracle
    w = W[name]
    say(f"[dense-full] {name}: generating")
    Q, K, V = synth.make_inputs(w)
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    say(f"[dense-full] {name}: kernel")
    O = lib.dense_attention(Qd, Kd, Vd)
    torch.cuda.synchronize()
    O = out_to_f64(O).reshape(-1, w.N, w.d)
    del Qd, Kd, Vd
    rng = np.random.default_rng(2)
    for z in (0, w.slices - 1):
        qsel = np.sort(rng.choice(w.N, size=128, replace=False))
        q64, k64, v64 = (slice_f64(x, w.dtype, z) for x in (Q, K, V))
        ref = oracle.full_attention(q64[qsel], k64, v64)
        err = np.abs(O[z][qsel] - ref).max()
        say(f"  slice {z}: max abs error {err:.3g}")
        assert err <= TOL_OUT[w.dtype], f"slice {z}: max abs error {err:.3g}"
