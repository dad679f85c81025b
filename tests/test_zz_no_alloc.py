"""mita_forward_noalloc (the entry point for callers that cannot allocate: the
library's fixed scratch array instead of a workspace) against mita_forward on the
same inputs, through the C ABI: bit-identical outputs on consecutive calls, the
later ones smaller (the scratch keeps the previous call's contents), and
problems beyond the scratch rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import say, to_device

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = [
    # bf16, s = 3 (partials and the combine kernel), ragged N
    W["tiny"].with_(name="na_bf16_s3", B=2, H=2, N=1000, grid_w=1000, pool_w=10, k=37, s=3, dtype="bf16"),
    # smaller, bf16, s = 1 (one-pass output kernel)
    W["tiny"].with_(name="na_bf16_s1", B=1, H=1, N=700, grid_w=700, pool_w=7, k=50, s=1, dtype="bf16"),
    # smaller again, fp32, d = 128, 2D grid
    W["tiny"].with_(name="na_f32_2d", B=1, H=1, N=16 * 20, grid_h=16, grid_w=20, pool_h=2, pool_w=4, d=128, k=40,
                    s=2),
]


def test_noalloc_matches_forward_on_consecutive_calls(lib):
    sizes = [w.slices * w.N * w.d for w in CASES]
    assert sizes == sorted(sizes, reverse=True)
    for w in CASES:
        say(f"[noalloc] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} k={w.k} s={w.s} {w.dtype}")
        Q, K, V = synth.make_inputs(w)
        Qd, Kd, Vd = (to_device(x, w.dtype) for x in (Q, K, V))
        grid, pool = (w.grid_h, w.grid_w), (w.pool_h, w.pool_w)
        ref = lib.Mita.create(Qd, w.m, w.k, w.s, grid=grid, pool=pool).forward(Qd, Kd, Vd)
        torch.cuda.synchronize()
        out = torch.full_like(Qd, float("nan"))
        lib.forward_noalloc(Qd, Kd, Vd, w.m, w.k, w.s, grid=grid, pool=pool, out=out)
        torch.cuda.synchronize()
        view = torch.int16 if w.dtype == "bf16" else torch.int32
        assert torch.equal(out.view(view), ref.view(view)), f"{w.name}: output differs from mita_forward"
        # a second call on the same inputs (scratch now holds this problem's state)
        out2 = lib.forward_noalloc(Qd, Kd, Vd, w.m, w.k, w.s, grid=grid, pool=pool)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(view), ref.view(view)), f"{w.name}: repeated call differs"


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    # ViT-B-like sizes need far more than 64 MiB of intermediates
    w = W["vit_b"]
    shape = lib.make_shape(w.B, w.H, w.N, w.d, w.m, "bf16", (w.grid_h, w.grid_w), (w.pool_h, w.pool_w))
    assert lib.workspace_bytes(shape, w.m, w.k, w.s) > lib.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000000)
    st = lib.load().mita_forward_noalloc(fake, fake, fake, w.m, w.k, w.s, fake, ctypes.byref(shape), None)
    assert st == lib.MITA_ERR_WORKSPACE
    assert "scratch" in lib.load().mita_last_error().decode()
