"""Python binding of libmita.so: argument marshalling only.

Every step runs in the library's HIP kernels; torch provides device memory and
the current stream. There is no fallback: if the library is missing, or a call
fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmita.so")

MITA_OK, MITA_ERR_INVALID_ARG, MITA_ERR_UNSUPPORTED, MITA_ERR_WORKSPACE, MITA_ERR_HIP = 0, -1, -2, -3, -4
MITA_F32, MITA_BF16 = 0, 1
SYMBOLS = ("mita_workspace_bytes", "mita_forward", "mita_pool", "mita_landmark", "mita_topk", "mita_route",
           "mita_gather", "mita_combine", "mita_dense_attention", "mita_forward_noalloc",
           "mita_backward_workspace_bytes", "mita_backward", "mita_status_string", "mita_last_error")
NOALLOC_SCRATCH_BYTES = 64 << 20   # MITA_NOALLOC_SCRATCH_BYTES


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "d", "grid_h", "grid_w", "pool_h", "pool_w", "dtype")]


class MitaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libmita.so (built in place by ``python -m sparse_top_routed_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_top_routed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz, sp = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER(Shape)
    lib.mita_workspace_bytes.argtypes = [sp, i, i, i]
    lib.mita_workspace_bytes.restype = sz
    lib.mita_forward.argtypes = [vp, vp, vp, i, i, i, vp, sp, vp, sz, vp]
    lib.mita_pool.argtypes = [vp, i, i, i, sp, vp, sz, vp, vp]
    lib.mita_landmark.argtypes = [vp, vp, i, i, i, sp, vp, sz, vp, vp, vp]
    lib.mita_topk.argtypes = [vp, i, i, i, sp, vp, sz, vp, vp]
    lib.mita_route.argtypes = [vp, i, i, i, sp, vp, sz, vp, vp]
    lib.mita_gather.argtypes = [vp, vp, vp, i, i, i, vp, sp, vp, sz, vp]
    lib.mita_combine.argtypes = [vp, i, i, i, vp, sp, vp, sz, vp]
    lib.mita_dense_attention.argtypes = [vp, vp, vp, vp, sp, vp]
    lib.mita_forward_noalloc.argtypes = [vp, vp, vp, i, i, i, vp, sp, vp]
    lib.mita_backward_workspace_bytes.argtypes = [sp, i, i, i]
    lib.mita_backward_workspace_bytes.restype = sz
    lib.mita_backward.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, vp, vp, sp, vp, sz, vp, sz, vp]
    for f in ("mita_forward", "mita_pool", "mita_landmark", "mita_topk", "mita_route", "mita_gather",
              "mita_combine", "mita_dense_attention", "mita_forward_noalloc", "mita_backward"):
        getattr(lib, f).restype = ctypes.c_int
    lib.mita_status_string.argtypes = [i]
    lib.mita_status_string.restype = ctypes.c_char_p
    lib.mita_last_error.argtypes = []
    lib.mita_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status == MITA_OK:
        return
    lib = load()
    msg = f"{lib.mita_status_string(status).decode()}: {lib.mita_last_error().decode()}"
    if status in (MITA_ERR_INVALID_ARG, MITA_ERR_UNSUPPORTED, MITA_ERR_WORKSPACE):
        raise ValueError(msg)
    raise MitaError(status, msg)


def make_shape(B: int, H: int, N: int, d: int, m: int, dtype, grid: Optional[Tuple[int, int]] = None,
               pool: Optional[Tuple[int, int]] = None) -> Shape:
    """Shape descriptor; ``grid``/``pool`` default to a 1D sequence pooled to m cells."""
    gh, gw = grid if grid is not None else (1, N)
    ph, pw = pool if pool is not None else (1, m)
    dt = MITA_BF16 if dtype in (torch.bfloat16, "bf16", MITA_BF16) else MITA_F32
    return Shape(B, H, N, d, gh, gw, ph, pw, dt)


def workspace_bytes(shape: Shape, m: int, k: int, s: int) -> int:
    n = load().mita_workspace_bytes(ctypes.byref(shape), m, k, s)
    if n == 0:
        raise ValueError(load().mita_last_error().decode())
    return n


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclass
class Mita:
    """One problem (shape and m, k, s) with its workspace; runs the whole pass or
    its steps (which must be called in order: pool, landmark, topk, route, gather,
    combine; ``output`` runs the last two)."""
    shape: Shape
    m: int
    k: int
    s: int
    workspace: torch.Tensor
    bwd_workspace: Optional[torch.Tensor] = None

    @classmethod
    def create(cls, Q: torch.Tensor, m: int, k: int, s: int, grid=None, pool=None) -> "Mita":
        if Q.dim() != 4:
            raise ValueError("Q must be [B, H, N, d]")
        B, H, N, d = Q.shape
        shape = make_shape(B, H, N, d, m, Q.dtype, grid, pool)
        ws = torch.empty(workspace_bytes(shape, m, k, s), dtype=torch.uint8, device=Q.device)
        return cls(shape, m, k, s, ws)

    # ------------------------------------------------------------------ checks
    def _inputs(self, *ts: torch.Tensor) -> None:
        want = torch.bfloat16 if self.shape.dtype == MITA_BF16 else torch.float32
        sh = (self.shape.B, self.shape.H, self.shape.N, self.shape.d)
        for t in ts:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if t.dtype != want or tuple(t.shape) != sh or not t.is_contiguous():
                raise ValueError(f"expected a contiguous {want} tensor of shape {sh}, got {t.dtype} {tuple(t.shape)}")

    def _ws(self):
        return ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel()

    # ------------------------------------------------------------------ calls
    def forward(self, Q, K, V, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        self._inputs(Q, K, V)
        out = torch.empty_like(Q) if out is None else out
        self._inputs(out)
        ws, n = self._ws()
        _check(load().mita_forward(_ptr(Q), _ptr(K), _ptr(V), self.m, self.k, self.s, _ptr(out),
                                   ctypes.byref(self.shape), ws, n, _stream()))
        return out

    def pool(self, Q, want: bool = False):
        self._inputs(Q)
        sh = self.shape
        Qt = torch.empty((sh.B, sh.H, self.m, sh.d), dtype=torch.float64, device=Q.device) if want else None
        ws, n = self._ws()
        _check(load().mita_pool(_ptr(Q), self.m, self.k, self.s, ctypes.byref(sh), ws, n, _ptr(Qt), _stream()))
        return Qt

    def landmark(self, K, V, want_vt: bool = False, want_s: bool = False):
        self._inputs(K, V)
        sh = self.shape
        Vt = torch.empty((sh.B, sh.H, self.m, sh.d), dtype=torch.float32, device=K.device) if want_vt else None
        S = torch.empty((sh.B, sh.H, self.m, sh.N), dtype=torch.float32, device=K.device) if want_s else None
        ws, n = self._ws()
        _check(load().mita_landmark(_ptr(K), _ptr(V), self.m, self.k, self.s, ctypes.byref(sh), ws, n, _ptr(Vt),
                                    _ptr(S), _stream()))
        return Vt, S

    def topk(self, K, want: bool = False):
        self._inputs(K)
        sh = self.shape
        I = torch.empty((sh.B, sh.H, self.m, self.k), dtype=torch.int32, device=K.device) if want else None
        ws, n = self._ws()
        _check(load().mita_topk(_ptr(K), self.m, self.k, self.s, ctypes.byref(sh), ws, n, _ptr(I), _stream()))
        return I

    def route(self, Q, want: bool = False):
        self._inputs(Q)
        sh = self.shape
        E = torch.empty((sh.B, sh.H, sh.N, self.s), dtype=torch.int32, device=Q.device) if want else None
        ws, n = self._ws()
        _check(load().mita_route(_ptr(Q), self.m, self.k, self.s, ctypes.byref(sh), ws, n, _ptr(E), _stream()))
        return E

    def gather(self, Q, K, V, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Routed part of step 5 (writes ``out`` itself only when the landmark part is fused)."""
        self._inputs(Q, K, V)
        out = torch.empty_like(Q) if out is None else out
        self._inputs(out)
        ws, n = self._ws()
        _check(load().mita_gather(_ptr(Q), _ptr(K), _ptr(V), self.m, self.k, self.s, _ptr(out),
                                  ctypes.byref(self.shape), ws, n, _stream()))
        return out

    def combine(self, Q, out: torch.Tensor) -> torch.Tensor:
        """Landmark part and merge of step 5 into ``out`` (after ``gather`` with the same ``out``)."""
        self._inputs(Q, out)
        ws, n = self._ws()
        _check(load().mita_combine(_ptr(Q), self.m, self.k, self.s, _ptr(out), ctypes.byref(self.shape), ws, n,
                                   _stream()))
        return out

    def output(self, Q, K, V, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Both parts of step 5."""
        return self.combine(Q, self.gather(Q, K, V, out))

    def backward(self, Q, K, V, out, dout, grads=None):
        """dQ, dK, dV (fp32) of sum(dout * out) for the forward this workspace holds
        (bf16 only); ``grads`` may give the three output tensors."""
        self._inputs(Q, K, V, out, dout)
        sh = self.shape
        if self.bwd_workspace is None:
            n = load().mita_backward_workspace_bytes(ctypes.byref(sh), self.m, self.k, self.s)
            if n == 0:
                raise ValueError(load().mita_last_error().decode())
            self.bwd_workspace = torch.empty(n, dtype=torch.uint8, device=Q.device)
        if grads is None:
            grads = tuple(torch.empty(Q.shape, dtype=torch.float32, device=Q.device) for _ in range(3))
        dQ, dK, dV = grads
        for g_ in grads:
            if g_.dtype != torch.float32 or g_.shape != Q.shape or not g_.is_contiguous():
                raise ValueError("gradients must be contiguous fp32 tensors shaped like Q")
        ws, n = self._ws()
        _check(load().mita_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), _ptr(dout), self.m, self.k, self.s,
                                    _ptr(dQ), _ptr(dK), _ptr(dV), ctypes.byref(sh), ws, n,
                                    ctypes.c_void_p(self.bwd_workspace.data_ptr()), self.bwd_workspace.numel(),
                                    _stream()))
        return dQ, dK, dV


def forward(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, m: int, k: int, s: int, grid=None, pool=None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MiTA attention forward: Q, K, V [B, H, N, d] (bf16 or fp32) on the GPU."""
    return Mita.create(Q, m, k, s, grid, pool).forward(Q, K, V, out)


def forward_noalloc(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, m: int, k: int, s: int, grid=None,
                    pool=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MiTA forward through mita_forward_noalloc: no workspace, the library's fixed
    scratch array instead (small problems only; calls on one GPU must not overlap)."""
    if Q.dim() != 4:
        raise ValueError("Q must be [B, H, N, d]")
    B, H, N, d = Q.shape
    shape = make_shape(B, H, N, d, m, Q.dtype, grid, pool)
    for t in (K, V):
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K and V must have one shape and dtype")
    for t in (Q, K, V):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
    if out is None:
        out = torch.empty_like(Q)
    elif out.shape != Q.shape or out.dtype != Q.dtype or not out.is_contiguous():
        raise ValueError("out must match Q")
    _check(load().mita_forward_noalloc(_ptr(Q), _ptr(K), _ptr(V), m, k, s, _ptr(out), ctypes.byref(shape),
                                       _stream()))
    return out


def dense_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Full softmax attention softmax(Q K^T / sqrt d) V over all N keys (the
    quadratic baseline MiTA is compared with): Q, K, V [B, H, N, d], bf16 or
    fp32, contiguous, on the GPU."""
    if Q.dim() != 4:
        raise ValueError("Q must be [B, H, N, d]")
    B, H, N, d = Q.shape
    for t in (K, V):
        if t.shape != Q.shape or t.dtype != Q.dtype:
            raise ValueError("Q, K and V must have one shape and dtype")
    for t in (Q, K, V):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous and on the GPU")
    if Q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty_like(Q)
    elif out.shape != Q.shape or out.dtype != Q.dtype or not out.is_contiguous():
        raise ValueError("out must match Q")
    shape = make_shape(B, H, N, d, 1, Q.dtype)
    _check(load().mita_dense_attention(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), ctypes.byref(shape), _stream()))
    return out
