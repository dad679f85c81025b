"""Seeded synthetic Q, K, V for the MiTA attention forward pass.

This module draws inputs only. It holds no step of the attention method, so the
fp64 oracle and the GPU path can both take their inputs from here without
sharing any of the method's arithmetic.

Recipe (the pages give no statistics of Q, K, V; these stand in for the image,
segmentation and long-sequence workloads the MiTA pages evaluate on):

* one numpy PCG64 stream per (batch, head) slice, seeded with
  ``SeedSequence([seed, b, h])``, so any slice can be drawn on its own;
* per slice, in this order: ``ncl`` cluster centres ``C ~ N(0, I_d)``, one label
  ``z_n ~ U{0..ncl-1}`` per token, then ``eps_Q, eps_K, eps_V ~ N(0, 1)`` of
  shape ``[N, d]``, then the needle token ids (``round(needle_frac * N)`` ids
  drawn without replacement);
* ``Q_n = alpha * C[z_n] + eps_Q``, likewise ``K`` and ``V`` with the same label;
* needle keys are scaled by ``needle_scale`` (keys only);
* all draws are float32; bf16 workloads are rounded to bfloat16 with
  round-to-nearest-even and held as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    grid_h: int
    grid_w: int
    pool_h: int
    pool_w: int
    k: int
    s: int
    dtype: str          # "f32" or "bf16"
    ncl: int
    alpha: float
    needle_frac: float = 0.0
    needle_scale: float = 4.0

    @property
    def m(self) -> int:
        return self.pool_h * self.pool_w

    @property
    def slices(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny fp32 case, a ViT-B-like image case (56x56 tokens
# pooled to 8x8), a segmentation-like case (128x128 pooled to 16x16), a long
# 1D sequence and a very long 1D sequence, the last two with 1 % needle keys.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 1024, 64, 1, 1024, 1, 16, 64, 1, "f32", 16, 0.3),
    "vit_b": Workload("vit_b", 32, 12, 3136, 64, 56, 56, 8, 8, 64, 1, "bf16", 64, 0.5),
    "seg": Workload("seg", 8, 12, 16384, 64, 128, 128, 16, 16, 128, 2, "bf16", 64, 0.5),
    "long": Workload("long", 2, 16, 65536, 128, 1, 65536, 1, 256, 256, 2, "bf16", 64, 0.5, 0.01),
    "very_long": Workload("very_long", 1, 8, 262144, 128, 1, 262144, 1, 512, 512, 4, "bf16", 64, 0.5, 0.01),
}


# Inference-time settings of (m, k, s) on the ViT-B-like inputs: the pages note
# that a model can be run with more landmarks or larger experts than it was
# trained with. m comes from the pooling grid of the 56 x 56 tokens (4x4, 7x7,
# 8x8, 14x14); every other field stays that of "vit_b".
SWEEP: Tuple[Tuple[int, int, int, int], ...] = (
    # (pool_h, pool_w, k, s)
    (4, 4, 64, 1),
    (7, 7, 64, 1),
    (8, 8, 32, 1),
    (8, 8, 64, 1),
    (8, 8, 128, 1),
    (8, 8, 256, 1),
    (8, 8, 64, 2),
    (8, 8, 64, 4),
    (14, 14, 64, 1),
    (14, 14, 128, 2),
)


def sweep_workloads(base: str = "vit_b") -> Sequence[Workload]:
    """The SWEEP settings applied to a base workload."""
    w = WORKLOADS[base]
    return [w.with_(name=f"{base}_m{ph * pw}_k{k}_s{s}", pool_h=ph, pool_w=pw, k=k, s=s) for ph, pw, k, s in SWEEP]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored input bits (bf16 as uint16, or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def draw_slice(w: Workload, b: int, h: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Draw one (b, h) slice: Q, K, V of shape [N, d] in float32 (before any bf16 rounding)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, b, h]))
    N, d = w.N, w.d
    C = rng.standard_normal((w.ncl, d), dtype=np.float32)
    z = rng.integers(0, w.ncl, size=N)
    centre = np.float32(w.alpha) * C[z]
    Q = centre + rng.standard_normal((N, d), dtype=np.float32)
    K = centre + rng.standard_normal((N, d), dtype=np.float32)
    V = centre + rng.standard_normal((N, d), dtype=np.float32)
    n_needles = int(round(w.needle_frac * N))
    if n_needles:
        ids = rng.choice(N, size=n_needles, replace=False)
        K[ids] *= np.float32(w.needle_scale)
    return Q, K, V


def make_inputs(w: Workload, seed: int = 0, slices: Optional[Sequence[Tuple[int, int]]] = None):
    """Q, K, V for the whole workload ([B, H, N, d]) or, when ``slices`` is given,
    for just those (b, h) pairs stacked as [len(slices), N, d].

    bf16 workloads come back as uint16 bit patterns, f32 ones as float32.
    """
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)] if slices is None else list(slices)
    store = np.uint16 if w.dtype == "bf16" else np.float32
    out = [np.empty((len(pairs), w.N, w.d), dtype=store) for _ in range(3)]
    for j, (b, h) in enumerate(pairs):
        for dst, x in zip(out, draw_slice(w, b, h, seed)):
            dst[j] = f32_to_bf16_bits(x) if w.dtype == "bf16" else x
    if slices is None:
        out = [x.reshape(w.B, w.H, w.N, w.d) for x in out]
    return tuple(out)
