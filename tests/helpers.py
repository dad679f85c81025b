"""Shared pieces of the GPU parity tests: run the library step by step on the
GPU, run the oracle on the same input bits, compare."""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import oracle
import synth

# Output tolerances (max abs error) for bf16 and fp32 inputs.
TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}
# Shared-expert tolerance: bf16 rounds the softmax weights and V~ operands to bf16.
TOL_VT = {"bf16": 1e-2, "f32": 2e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu_steps(w: synth.Workload, Q, K, V, lib, want_s: bool = True) -> Dict[str, np.ndarray]:
    """Run pool, landmark, topk, route and gather through the C ABI; return the
    intermediates and the output as numpy arrays."""
    Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
    call = lib.Mita.create(Qd, w.m, w.k, w.s, grid=(w.grid_h, w.grid_w), pool=(w.pool_h, w.pool_w))
    Qt = call.pool(Qd, want=True)
    Vt, S = call.landmark(Kd, Vd, want_vt=True, want_s=want_s)
    I = call.topk(Kd, want=True)
    E = call.route(Qd, want=True)
    O = call.output(Qd, Kd, Vd)
    torch.cuda.synchronize()
    res = {"Qt": Qt.cpu().numpy(), "Vt": Vt.cpu().numpy().astype(np.float64), "I": I.cpu().numpy(),
           "E": E.cpu().numpy(), "O": out_to_f64(O)}
    if want_s:
        res["S"] = S.cpu().numpy().astype(np.float64)
    return res


def slice_f64(x: np.ndarray, dtype: str, z: int) -> np.ndarray:
    """fp64 copy of slice z of a [B, H, N, d] (or [BH, N, d]) input array."""
    flat = x.reshape(-1, x.shape[-2], x.shape[-1])
    return synth.to_f64(flat[z], dtype)


def check_slice(w: synth.Workload, Q, K, V, gpu: Dict[str, np.ndarray], z: int,
                queries: Optional[Sequence[int]] = None, check_s: bool = True,
                route_all: bool = False, near_margin: int = 0) -> Dict[str, float]:
    """Compare slice z of the GPU results with the oracle. Raises AssertionError on
    a parity failure and returns a few statistics.

    queries: the queries whose routing and output are checked (all when None).
    route_all: check the routing of every query of the slice, and the output on
    `queries` plus the `near_margin` queries whose routing margin is smallest."""
    q64, k64, v64 = (slice_f64(x, w.dtype, z) for x in (Q, K, V))
    d = w.d
    Qt = oracle.pool(q64, w.grid_h, w.grid_w, w.pool_h, w.pool_w)
    g_qt = gpu["Qt"].reshape(-1, w.m, d)[z]
    rel_qt = np.abs(g_qt - Qt).max() / max(np.abs(Qt).max(), 1e-300)
    assert rel_qt <= 1e-12, f"slice {z}: landmark queries off by {rel_qt:.3g} (relative)"

    S = oracle.scores(Qt, k64)
    if check_s and "S" in gpu:
        # the score rows must honour the error bound the exact selection relies on
        g_s = gpu["S"].reshape(-1, w.m, w.N)[z]
        kmax = np.sqrt((k64 ** 2).sum(axis=1)).max()
        qn = np.sqrt((Qt ** 2).sum(axis=1))
        u = 2.0 ** -23
        gamma = (2 ** -16 + (2 * d + 4) * u) if w.dtype == "bf16" else (u + (d + 4) * u)
        bound = gamma * qn[:, None] * kmax
        diff = np.abs(g_s - S)
        excess = np.where(bound > 0, diff / np.where(bound > 0, bound, 1.0), np.where(diff > 0, np.inf, 0.0)).max()
        assert excess <= 1.0, f"slice {z}: score error {excess:.3g} x the bound"

    Vt = oracle.shared_expert(Qt, k64, v64)
    g_vt = gpu["Vt"].reshape(-1, w.m, d)[z]
    err_vt = np.abs(g_vt - Vt).max()
    assert err_vt <= TOL_VT[w.dtype], f"slice {z}: shared expert max abs error {err_vt:.3g}"

    g_I = gpu["I"].reshape(-1, w.m, w.k)[z].astype(np.int64)
    assert (np.diff(g_I, axis=1) > 0).all(), f"slice {z}: expert index lists not strictly ascending"
    ok_I = oracle.valid_topk_sets(S, g_I, w.k)
    assert ok_I.all(), f"slice {z}: {np.count_nonzero(~ok_I)} invalid expert sets (rows {np.nonzero(~ok_I)[0][:8]})"
    I_or = oracle.topk_experts(S, w.k)
    margins = oracle.topk_margins(S, w.k)
    exact_rows = (g_I == I_or).all(axis=1)
    assert exact_rows[margins >= 1e-6].all(), f"slice {z}: an expert set differs on a row with a clear margin"

    N = w.N
    qsel = np.arange(N) if queries is None else np.asarray(queries)
    rsel = np.arange(N) if route_all else qsel
    R = oracle.route_scores(q64[rsel], Qt)
    g_E = gpu["E"].reshape(-1, N, w.s)[z].astype(np.int64)
    ok_E = oracle.valid_route_sets(R, g_E[rsel], w.s)
    assert ok_E.all(), f"slice {z}: {np.count_nonzero(~ok_E)} invalid routings (queries {rsel[~ok_E][:8]})"
    E_or = oracle.route(q64[rsel], Qt, w.s)
    rmarg = oracle.route_margins(R, w.s)
    del R
    same_E = (np.sort(g_E[rsel], axis=1) == np.sort(E_or, axis=1)).all(axis=1)
    assert same_E[rmarg >= 1e-6].all(), f"slice {z}: a routing differs on a query with a clear margin"
    if near_margin:   # the output of the queries nearest a routing tie is checked too
        qsel = np.union1d(qsel, rsel[np.argsort(rmarg, kind="stable")[:near_margin]])

    # output, recomputed by the oracle with the GPU's (validated) sets
    O = oracle.attend(q64, k64, v64, Qt, Vt, g_I, g_E, qsel)
    g_O = gpu["O"].reshape(-1, N, d)[z][qsel]
    err_o = np.abs(g_O - O).max()
    assert err_o <= TOL_OUT[w.dtype], f"slice {z}: output max abs error {err_o:.3g}"
    return {"qt_rel": rel_qt, "vt_err": err_vt, "out_err": err_o, "I_exact_rows": float(exact_rows.mean()),
            "E_exact": float(same_E.mean())}
