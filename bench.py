"""MiTA attention forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_b]

Prints one JSON line: query-tokens/s of the whole forward pass (B*H*N per call)
on seeded synthetic inputs resident in HBM, the roofline position of the
dominant kernel (timed live with HIP events on the library's stream) and the
fp64 CPU oracle timed on a bounded sample of the same workload.
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


def step_bytes(w) -> dict:
    """Algorithmic HBM bytes per forward call, by step (each input or
    intermediate counted once per step that must read or write it)."""
    e = 2 if w.dtype == "bf16" else 4
    BH, N, d, m, k, s = w.slices, w.N, w.d, w.m, w.k, w.s
    tok = BH * N * d * e
    nblk = -(-N // 64)
    nbg = nblk * (1 if nblk >= 4 * k else (4 if 4 * nblk >= k else 16))   # group maxima per row (64, 16 or 4 scores)
    return {
        "pool": tok + BH * m * d * (8 + 4 + 4),
        # K and V read once, group maxima of the score rows written once
        "landmark": 2 * tok + BH * m * nbg * 4,
        # group maxima read, K read once more (candidate pass), expert lists written
        "topk": BH * m * nbg * 4 + tok + BH * m * k * 4,
        "route": tok + BH * N * s * 4,
        # Q read, each expert's k gathered K/V rows once, output written, + the per-slot partials
        # written and read back when s > 1 or m > 64 (d values in 16 bits for bf16, else 32, and
        # 16 bytes of (max, sum, scale))
        "gather": 2 * tok + BH * m * k * d * e * 2
        + (BH * N * s * (d * e + 16) * 2 if (s > 1 or m > 64) else 0),
    }


# Kernel sources each step's dominant kernel is built from: a stored traffic
# figure is only reported while these files are byte-identical to the ones it
# was measured on.
KERNEL_SOURCES = {
    "gather": ["sparse_top_routed_amd/csrc/gather.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "topk": ["sparse_top_routed_amd/csrc/topk.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "route": ["sparse_top_routed_amd/csrc/route.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "landmark": ["sparse_top_routed_amd/csrc/landmark.hip", "sparse_top_routed_amd/csrc/attn_core.h"],
    "pool": ["sparse_top_routed_amd/csrc/pool.hip"],
}
COMMON_SOURCES = ["sparse_top_routed_amd/csrc/common.h", "sparse_top_routed_amd/csrc/plan.h",
                  "sparse_top_routed_amd/build.py"]
KERNEL_NAMES = {
    "gather": "gather1_kernel", "topk": "topk_cand_kernel", "route": "route_fast_kernel",
    "landmark": "landmark_kernel", "pool": "pool_kernel",
}


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


def cpu_baseline(w, Q, K, V, budget_s: float = 12.0) -> dict:
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        for z in range(w.slices):
            q64, k64, v64 = (synth.to_f64(x.reshape(-1, w.N, w.d)[z], w.dtype) for x in (Q, K, V))
            oracle.forward(q64, k64, v64, w.grid_h, w.grid_w, w.pool_h, w.pool_w, w.k, w.s)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    return {"value": done * w.N / el, "unit": "query-tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.slices} (batch, head) slices of {w.name}, all {w.N} queries each, "
                      f"fp64 numpy, BLAS limited to 1 thread, {el:.1f} s"}


def step_times(call, Qd, Kd, Vd, out, steps: int) -> dict:
    """Mean time (ms) of each step entry point, the launches of one forward run one
    step at a time, bracketed by events on the stream the kernels run on."""
    import torch

    st = torch.cuda.current_stream()
    names = ["pool", "landmark", "topk", "route", "gather"]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    acc = dict.fromkeys(names, 0.0)
    for _ in range(steps):
        ev[0].record(st)
        call.pool(Qd); ev[1].record(st)
        call.landmark(Kd, Vd); ev[2].record(st)
        call.topk(Kd); ev[3].record(st)
        call.route(Qd); ev[4].record(st)
        call.gather(Qd, Kd, Vd, out); ev[5].record(st)
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU reaches its steady clocks only after some tens of ms of work: with 5
    # warm-up forwards (~3 ms) the timed forwards run ~12 % slower than after 100
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="vit_b")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--breakdown", action="store_true", help="print per-step times to stderr")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 elementwise copies of 512 MiB (read and write 2^29 bytes each), the "
                         "reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--print-sha", action="store_true", help="print the dominant kernels' source hashes and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="time the forward pass over the inference-time (m, k, s) settings of synth.SWEEP on the "
                         "workload's inputs (one JSON line per setting) instead of the benchmark line")
    ap.add_argument("--dense", action="store_true",
                    help="time the full-attention comparator against the MiTA forward on the workload's inputs "
                         "(one JSON line) instead of the benchmark line")
    a = ap.parse_args()
    if a.print_sha:
        for step in KERNEL_SOURCES:
            print(step, KERNEL_NAMES[step], sources_sha256(step))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MiTA forward here runs on a single MI355X "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from sparse_top_routed_amd import mita

    w = synth.WORKLOADS[a.workload]
    Q, K, V = synth.make_inputs(w)

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    Qd, Kd, Vd = dev(Q), dev(K), dev(V)
    if a.sweep:
        return sweep(w, Qd, Kd, Vd, a.steps, a.warmup, a.breakdown)
    if a.dense:
        return dense_compare(w, Qd, Kd, Vd, a.steps, a.warmup)
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

    # per-step times: the same launches as forward, one step entry point at a time
    names = ["pool", "landmark", "topk", "route", "gather"]
    per = step_times(call, Qd, Kd, Vd, out, a.steps)
    nbytes = step_bytes(w)
    dom = max(per, key=per.get)
    kname = KERNEL_NAMES[dom]
    if dom == "gather" and not (w.s == 1 and w.k <= 64 and w.m <= 64):
        # the one-pass kernel serves s = 1 with k, m <= 64 only
        kname = "gather_kernel" if w.s == 1 else "gather_kernel+combine_kernel"
    achieved = nbytes[dom] / (per[dom] * 1e-3) / 1e9
    if a.breakdown:
        for n in names:
            print(f"{n:9s} {per[n] * 1e3:9.1f} us  {nbytes[n] / (per[n] * 1e-3) / 1e9:8.1f} GB/s (algorithmic)",
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
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": stored_traffic(dom, w.name, kname), "algorithmic_bytes": nbytes[dom]},
        "step_ms": per,
    }
    if not a.no_cpu:
        res["cpu_baseline"] = cpu_baseline(w, Q, K, V)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
