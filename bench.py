"""MiTA attention forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload very_long]

Prints one JSON line: query-tokens/s of the whole forward pass (B*H*N per call)
on seeded synthetic inputs resident in HBM (default: the very long sequence,
B=1, H=8, N=262144, d=128, m=512, k=512, s=4, bf16), the roofline position of
the dominant kernel (timed live with HIP events on the library's stream; MFMA
fraction against the bf16 dense peak and HBM fraction beside it), the MFMA and
HBM fractions of every step, and the fp64 CPU oracle timed on the host's cores
over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MiTA fwd query-tokens/sec (B·H·N/s) + % bf16 MFMA peak, % HBM BW"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def _fused(w) -> bool:
    """Whether the routed-expert kernel also attends the landmark pairs and writes
    the output (s = 1 with m <= 64), so that the combine step launches nothing."""
    return w.s == 1 and w.m <= 64


def step_bytes(w) -> dict:
    """Algorithmic HBM bytes per forward call, by step (each input or
    intermediate counted once per step that must read or write it)."""
    e = 2 if w.dtype == "bf16" else 4
    ep = 2 if w.dtype == "bf16" else 4   # partial outputs: fp16 for bf16 inputs, else fp32
    BH, N, d, m, k, s = w.slices, w.N, w.d, w.m, w.k, w.s
    tok = BH * N * d * e
    nblk = -(-N // 64)
    nbg = nblk * (1 if nblk >= 4 * k else (4 if 4 * nblk >= k else 16))   # group maxima per row (64, 16 or 4 scores)
    partials = BH * N * s * (d * ep + 16)
    fused = _fused(w)
    return {
        "pool": tok + BH * m * d * (8 + 4 + 4),
        # K and V read once, group maxima of the score rows written once
        "landmark": 2 * tok + BH * m * nbg * 4,
        # group maxima read, K read once more (candidate pass), expert lists written
        "topk": BH * m * nbg * 4 + tok + BH * m * k * 4,
        "route": tok + BH * N * s * 4,
        # each query row read once per routed slot, each expert's k gathered K/V rows once, and the
        # output (fused) or the per-slot partials written
        "gather": BH * N * s * d * e + BH * m * k * d * e * 2 + (tok if fused else partials),
        # query rows and the partials read, the output written (the landmark pairs are m rows)
        "combine": 0 if fused else 2 * tok + partials,
    }


def step_flops(w) -> dict:
    """Algorithmic MFMA flops per forward call, by step (2 per multiply-add; the
    bf16 hi + lo split of Q~ that keeps scores fp32-accurate is not counted)."""
    BH, N, d, m, k, s = w.slices, w.N, w.d, w.m, w.k, w.s
    fused = _fused(w)
    return {
        "pool": 0,
        "landmark": 4 * BH * m * N * d,            # Q~ K^T and P V
        "topk": 2 * BH * m * N * d,                # Q~ K^T again (candidate pass)
        "route": 2 * BH * N * m * d,               # Q Q~^T
        "gather": 4 * BH * N * k * s * d + (4 * BH * N * m * d if fused else 0),
        "combine": 0 if fused else 4 * BH * N * m * d,
    }


# Kernel sources each step's dominant kernel is built from: a stored traffic
# figure is only reported while these files are byte-identical to the ones it
# was measured on.
KERNEL_SOURCES = {
    "gather": ["sparse_top_routed_amd/csrc/gather.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "combine": ["sparse_top_routed_amd/csrc/gather.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "topk": ["sparse_top_routed_amd/csrc/topk.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "route": ["sparse_top_routed_amd/csrc/route.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "landmark": ["sparse_top_routed_amd/csrc/landmark.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "pool": ["sparse_top_routed_amd/csrc/pool.hip"],
}
COMMON_SOURCES = ["sparse_top_routed_amd/csrc/common.h", "sparse_top_routed_amd/csrc/plan.h",
                  "sparse_top_routed_amd/build.py"]
STEPS = ["pool", "landmark", "topk", "route", "gather", "combine"]


def kernel_names(w) -> dict:
    """The kernel that does each step's arithmetic for this workload."""
    if _fused(w):
        gather = "gather1_kernel" if w.k <= 64 else "gather_kernel"
    else:   # partials: the direct-load kernel for bf16 inputs
        gather = "gatherd_kernel" if w.dtype == "bf16" else "gather_kernel"
    direct = w.dtype == "bf16" and w.m > 64   # several landmark tiles: the direct-load kernels
    return {"pool": "pool_kernel", "landmark": "landmarkd_kernel" if direct else "landmark_kernel",
            "topk": "topk_candd_kernel" if direct else "topk_cand_kernel",
            "route": "route_fast_kernel" if w.m <= 64 else "route_multi_kernel", "gather": gather,
            "combine": "combined_kernel" if w.dtype == "bf16" else "combine_kernel"}


def sources_sha256(step: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[step] + COMMON_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic(step: str, workload: str, kernel: str):
    """HBM bytes per launch of the step's dominant kernel, from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summary under profiles/, or None when there is none
    or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                key, val = line[2:].split(": ", 1)
                vals[key.strip()] = val.strip().strip("`")
    if vals.get("source_sha256") != sources_sha256(step):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)   # one BLAS thread per process: the processes are the parallelism


def _cpu_slice(w, z):
    import synth
    b, h = divmod(z, w.H)
    Q, K, V = synth.make_inputs(w, slices=[(b, h)])
    return tuple(synth.to_f64(x[0], w.dtype) for x in (Q, K, V))


def _cpu_fixed(args):
    """Per-slice part of the oracle (pooling, shared expert, expert sets): its time
    and the small results the per-query part needs (input generation untimed)."""
    import oracle
    w, z = args
    q64, k64, v64 = _cpu_slice(w, z)
    t0 = time.perf_counter()
    Qt = oracle.pool(q64, w.grid_h, w.grid_w, w.pool_h, w.pool_w)
    S = oracle.scores(Qt, k64)
    Vt = oracle.shared_expert(Qt, k64, v64)
    I = oracle.topk_experts(S, w.k)
    return z, time.perf_counter() - t0, Qt, Vt, I


def _cpu_queries(args):
    """Per-query part of the oracle (routing, output) for a sample of queries."""
    import numpy as np
    import oracle
    w, z, qs, Qt, Vt, I = args
    q64, k64, v64 = _cpu_slice(w, z)
    t0 = time.perf_counter()
    E = np.full((w.N, w.s), -1, dtype=np.int64)
    E[qs] = oracle.route(q64[qs], Qt, w.s)
    oracle.attend(q64, k64, v64, Qt, Vt, I, E, qs)
    return z, len(qs), time.perf_counter() - t0


def cpu_baseline(w, workers: int, queries_per_slice: int = 4096) -> dict:
    """The fp64 oracle as it stands on the host's cores: one single-threaded process
    per core (at most 16, the CPU share of one GPU on the box). The per-slice part
    runs whole on up to 2 x workers slices; the per-query part on a sample of
    queries of each of them, in chunks spread over all workers. Each task is
    timed inside its process while all processes run (so memory contention is
    included); the whole-job time is estimated as the summed task times, scaled
    to all slices and queries, divided by the number of processes (perfect load
    balance, which favours the CPU)."""
    import multiprocessing as mp

    import numpy as np

    nslice = min(w.slices, 2 * workers)
    zs = [int(z) for z in np.linspace(0, w.slices - 1, nslice).round().astype(int)]
    zs = sorted(set(zs))
    ctx = mp.get_context("spawn")
    wall0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        fixed = pool.map(_cpu_fixed, [(w, z) for z in zs], chunksize=1)
        rng = np.random.default_rng(3)
        tasks = []
        for z, _, Qt, Vt, I in fixed:
            qs = np.sort(rng.choice(w.N, size=min(w.N, queries_per_slice), replace=False))
            for c in np.array_split(qs, max(1, len(qs) // 512)):
                tasks.append((w, z, c, Qt, Vt, I))
        per_q = pool.map(_cpu_queries, tasks, chunksize=1)
    wall = time.perf_counter() - wall0
    t_fixed = sum(f[1] for f in fixed) / len(fixed)                     # per slice
    nq = sum(p[1] for p in per_q)
    t_query = sum(p[2] for p in per_q) / nq                             # per query
    t_slice = t_fixed + w.N * t_query
    t_job = w.slices * t_slice / workers
    nproc = os.cpu_count()
    return {"value": w.slices * w.N / t_job, "unit": "query-tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(), "nproc": nproc,
            "sample": f"{w.name}: per-slice part (pool, shared expert, expert sets) whole on {len(zs)} of "
                      f"{w.slices} slices ({t_fixed:.2f} s each), per-query part (routing, output) on {nq} "
                      f"sampled queries ({t_query * 1e6:.1f} us each); fp64 numpy, {workers} single-threaded "
                      f"processes, job time = {w.slices} slices x {t_slice:.2f} s / {workers}; {wall:.1f} s wall"}


def step_times(call, Qd, Kd, Vd, out, steps: int) -> dict:
    """Mean time (ms) of each step entry point, the launches of one forward run one
    step at a time, bracketed by events on the stream the kernels run on."""
    import torch

    st = torch.cuda.current_stream()
    names = STEPS
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = dict.fromkeys(names, 0.0)
    for _ in range(steps):
        ev[0].record(st)
        call.pool(Qd); ev[1].record(st)
        call.landmark(Kd, Vd); ev[2].record(st)
        call.topk(Kd); ev[3].record(st)
        call.route(Qd); ev[4].record(st)
        call.gather(Qd, Kd, Vd, out); ev[5].record(st)
        call.combine(Qd, out); ev[6].record(st)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    return {n: acc[n] / steps for n in names}


def sweep(w, Qd, Kd, Vd, steps: int, warmup: int, breakdown: bool) -> int:
    """Forward throughput for each (m, k, s) setting of synth.SWEEP on the same
    inputs; per-setting parity is covered by the GPU tests."""
    import torch

    import synth
    from sparse_top_routed_amd import mita

    st = torch.cuda.current_stream()
    for v in synth.sweep_workloads(w.name):
        call = mita.Mita.create(Qd, v.m, v.k, v.s, grid=(v.grid_h, v.grid_w), pool=(v.pool_h, v.pool_w))
        out = torch.empty_like(Qd)
        for _ in range(warmup):
            call.forward(Qd, Kd, Vd, out)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(st)
        for _ in range(steps):
            call.forward(Qd, Kd, Vd, out)
        t1.record(st)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        res = {"workload": v.name, "m": v.m, "k": v.k, "s": v.s, "ms_per_step": ms,
               "value": v.slices * v.N / (ms * 1e-3), "unit": "query-tokens/s", "keys_per_query": v.m + v.k * v.s}
        if breakdown:
            res["step_ms"] = step_times(call, Qd, Kd, Vd, out, steps)
        print(json.dumps(res), flush=True)
        del call, out
    return 0


def dense_compare(w, Qd, Kd, Vd, steps: int, warmup: int) -> int:
    """The full-attention comparator (softmax over all N keys, the quadratic
    baseline) against the MiTA forward on the same inputs: mean time of each and
    the ratio, plus the comparator's MFMA throughput (4 N^2 d flops per slice)."""
    import torch

    from sparse_top_routed_amd import mita

    st = torch.cuda.current_stream()
    call = mita.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    out, dout = torch.empty_like(Qd), torch.empty_like(Qd)

    def timed(fn, n):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(st)
        for _ in range(n):
            fn()
        t1.record(st)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    for _ in range(warmup):
        call.forward(Qd, Kd, Vd, out)
    mita_ms = timed(lambda: call.forward(Qd, Kd, Vd, out), steps)
    first = timed(lambda: mita.dense_attention(Qd, Kd, Vd, dout), 1)   # warm-up; sizes the timed run to ~2 s
    n = max(1, min(steps, int(2000.0 / max(first, 1e-3))))
    dense_ms = timed(lambda: mita.dense_attention(Qd, Kd, Vd, dout), n)
    flops = 4.0 * w.slices * w.N * w.N * w.d
    peak = 2500.0 if w.dtype == "bf16" else 157.3   # dense MFMA TFLOP/s of the input dtype
    tf = flops / (dense_ms * 1e-3) / 1e12
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m, "k": w.k, "s": w.s,
           "dtype": w.dtype, "mita_ms": mita_ms, "mita_steps": steps, "dense_ms": dense_ms, "dense_steps": n,
           "speedup": dense_ms / mita_ms, "keys_per_query": {"mita": w.m + w.k * w.s, "dense": w.N},
           "dense_tflops": tf, "dense_mfma_frac": tf / peak}
    print(json.dumps(res), flush=True)
    return 0


def backward_bench(w, Qd, Kd, Vd, steps: int, warmup: int) -> int:
    """Forward and backward (mita_backward: dQ, dK, dV of sum(dout * out), expert sets
    and routing held fixed) on the workload's inputs: mean time of each with HIP
    events on the library's stream, and the backward's algorithmic MFMA rate: 5
    contractions per (query, key) pair (scores recomputed, dO V^T, dS K, dS^T Q,
    P^T dO), 10 d flops per pair, over the routed pairs (N k s per slice) and the
    landmark pairs of the final attention and of the shared expert (N m each)."""
    import torch

    from sparse_top_routed_amd import mita

    if w.dtype != "bf16":
        print("the backward supports bf16 inputs only", file=sys.stderr)
        return 2
    st = torch.cuda.current_stream()
    call = mita.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    out = torch.empty_like(Qd)
    dout = torch.randn(Qd.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(3)).to(torch.bfloat16)
    grads = tuple(torch.empty(Qd.shape, dtype=torch.float32, device="cuda") for _ in range(3))
    for _ in range(warmup):
        call.forward(Qd, Kd, Vd, out)
        call.backward(Qd, Kd, Vd, out, dout, grads)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd = bwd = 0.0
    for _ in range(steps):
        ev[0].record(st)
        call.forward(Qd, Kd, Vd, out)
        ev[1].record(st)
        call.backward(Qd, Kd, Vd, out, dout, grads)
        ev[2].record(st)
        torch.cuda.synchronize()
        fwd += ev[0].elapsed_time(ev[1])
        bwd += ev[1].elapsed_time(ev[2])
    fwd, bwd = fwd / steps, bwd / steps
    flops = 10.0 * w.slices * w.d * (w.N * w.k * w.s + 2 * w.N * w.m)
    tf = flops / (bwd * 1e-3) / 1e12
    res = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m, "k": w.k, "s": w.s,
           "dtype": w.dtype, "steps": steps, "warmup": warmup, "forward_ms": fwd, "backward_ms": bwd,
           "fwd_bwd_query_tokens_per_s": w.slices * w.N / ((fwd + bwd) * 1e-3),
           "backward_algorithmic_tflop": flops / 1e12, "backward_tflops": tf,
           "backward_mfma_frac": tf / BF16_PEAK_TFLOPS}
    print(json.dumps(res), flush=True)
    return 0


def _cpu_workers(requested: int) -> int:
    have = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(requested or have, have, 16))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clocks only after some tens of ms of work (a very long
    # forward is ~10 ms, so a few warm-up forwards suffice; small workloads need more)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="very_long")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the CPU baseline (default: the usable cores, at most 16)")
    ap.add_argument("--breakdown", action="store_true", help="print per-step times to stderr")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 elementwise copies of 512 MiB (read and write 2^29 bytes each), the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--print-sha", action="store_true", help="print the dominant kernels' source hashes and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="time the forward pass over the inference-time (m, k, s) settings of synth.SWEEP on the "
                         "workload's inputs (one JSON line per setting) instead of the benchmark line; the settings "
                         "are pooling grids of the ViT-B-like workload, which it uses unless --workload names another "
                         "2D-grid workload")
    ap.add_argument("--backward", action="store_true",
                    help="time the forward and the backward (mita_backward) on the workload's inputs (one JSON line) "
                         "instead of the benchmark line")
    ap.add_argument("--dense", action="store_true",
                    help="time the full-attention comparator against the MiTA forward on the workload's inputs "
                         "(one JSON line) instead of the benchmark line")
    a = ap.parse_args()
    if a.print_sha:
        for step in KERNEL_SOURCES:
            print(step, sources_sha256(step))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MiTA forward here runs on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np

    import synth

    if a.sweep and a.workload == ap.get_default("workload"):
        a.workload = "vit_b"
    w = synth.WORKLOADS[a.workload]
    # the CPU baseline runs first, before anything touches the GPU: its worker
    # processes start from a clean interpreter and never share the GPU timing
    cpu = None
    if not (a.no_cpu or a.sweep or a.dense or a.backward):
        cpu = cpu_baseline(w, _cpu_workers(a.cpu_workers))

    import torch

    from sparse_top_routed_amd import mita

    Q, K, V = synth.make_inputs(w)

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    del Q, K, V
    if a.sweep:
        return sweep(w, Qd, Kd, Vd, a.steps, a.warmup, a.breakdown)
    if a.dense:
        return dense_compare(w, Qd, Kd, Vd, a.steps, a.warmup)
    if a.backward:
        return backward_bench(w, Qd, Kd, Vd, a.steps, a.warmup)
    call = mita.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    out = torch.empty_like(Qd)
    for _ in range(a.warmup):
        call.forward(Qd, Kd, Vd, out)
    torch.cuda.synchronize()

    st = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(st)
    for _ in range(a.steps):
        call.forward(Qd, Kd, Vd, out)
    t1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / a.steps
    tokens = w.slices * w.N

    # per-step times: the same launches as forward, one step entry point at a time,
    # events on the stream the library launches on (the current stream)
    per = step_times(call, Qd, Kd, Vd, out, a.steps)
    nbytes, nflops, names = step_bytes(w), step_flops(w), kernel_names(w)
    frac = {}
    for n in STEPS:
        if per[n] <= 0 or (nflops[n] == 0 and nbytes[n] == 0):
            continue
        sec = per[n] * 1e-3
        frac[n] = {"kernel": names[n], "ms": per[n],
                   "mfma_frac": nflops[n] / sec / 1e12 / BF16_PEAK_TFLOPS if w.dtype == "bf16" and nflops[n] else None,
                   "hbm_frac": nbytes[n] / sec / 1e9 / HBM_PEAK_GBS}
    dom = max((n for n in STEPS if n in frac), key=lambda n: per[n])
    sec = per[dom] * 1e-3
    # the binding roof by the roofline model: the larger of flops / peak and bytes / bandwidth
    t_mfma = nflops[dom] / (BF16_PEAK_TFLOPS * 1e12) if w.dtype == "bf16" else 0.0
    t_hbm = nbytes[dom] / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "kernel": names[dom], "achieved": nflops[dom] / sec / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": nflops[dom] / sec / 1e12 / BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "kernel": names[dom], "achieved": nbytes[dom] / sec / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": nbytes[dom] / sec / 1e9 / HBM_PEAK_GBS}
    roof.update({"traffic": stored_traffic(dom, w.name, names[dom]), "algorithmic_flops": nflops[dom],
                 "algorithmic_bytes": nbytes[dom], "hbm_frac": nbytes[dom] / sec / 1e9 / HBM_PEAK_GBS,
                 "ms": per[dom]})
    if a.breakdown:
        for n in STEPS:
            if n in frac:
                f = frac[n]
                mf = f"{f['mfma_frac'] * 100:5.1f} % MFMA" if f["mfma_frac"] is not None else " " * 12
                print(f"{n:9s} {per[n] * 1e3:9.1f} us  {mf}  {f['hbm_frac'] * 100:5.1f} % HBM  ({f['kernel']})",
                      file=sys.stderr)
        print(f"forward  {ms * 1e3:9.1f} us  wall {wall / a.steps * 1e6:9.1f} us", file=sys.stderr)
    if a.copy_calibration:
        src = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    res = {
        "metric": METRIC, "value": tokens / (ms * 1e-3), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m, "k": w.k, "s": w.s,
                   "grid": [w.grid_h, w.grid_w], "pool": [w.pool_h, w.pool_w]},
        "roofline": roof,
        "steps_roofline": frac,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
