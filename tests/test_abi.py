"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments before enqueueing
anything (no test here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from sparse_top_routed_amd import mita

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mita.h")
FAKE = 0x10000000   # 256-byte aligned, never dereferenced: every call below fails its checks first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mita_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mita.load()
    names = declared_functions()
    assert set(names) == set(mita.SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def shape(B=1, H=1, N=1024, d=64, gh=1, gw=1024, ph=1, pw=16, dt=mita.MITA_F32):
    return mita.Shape(B, H, N, d, gh, gw, ph, pw, dt)


def test_workspace_bytes_grows_with_problem():
    a = mita.workspace_bytes(shape(), 16, 64, 1)
    b = mita.workspace_bytes(shape(B=2), 16, 64, 1)
    c = mita.workspace_bytes(shape(), 16, 64, 2)
    assert 0 < a < b and a < c
    assert a % 256 == 0
    # the score rows alone are m * N fp32 values per slice
    assert a >= 16 * 1024 * 4


@pytest.mark.parametrize("sh,m,k,s,code", [
    (shape(N=1000), 16, 64, 1, mita.MITA_ERR_INVALID_ARG),          # grid does not cover N
    (shape(pw=8), 16, 64, 1, mita.MITA_ERR_INVALID_ARG),            # pool grid != m
    (shape(), 16, 2000, 1, mita.MITA_ERR_INVALID_ARG),              # k > N
    (shape(), 16, 0, 1, mita.MITA_ERR_INVALID_ARG),                 # k < 1
    (shape(), 16, 64, 17, mita.MITA_ERR_INVALID_ARG),               # s > m
    (shape(ph=2, pw=8, gh=1), 16, 64, 1, mita.MITA_ERR_INVALID_ARG),  # pool_h > grid_h
    (shape(d=96), 16, 64, 1, mita.MITA_ERR_UNSUPPORTED),            # head size
    (shape(dt=7), 16, 64, 1, mita.MITA_ERR_INVALID_ARG),            # dtype
    (shape(N=8192, gw=8192, pw=8192), 8192, 64, 1, mita.MITA_ERR_UNSUPPORTED),  # m above 4096
    (shape(N=8192, gw=8192, pw=96, dt=mita.MITA_BF16), 96, 32, 2, mita.MITA_ERR_UNSUPPORTED),  # bf16, m > 64, k < 64, N >= 256 k
])
def test_invalid_arguments(sh, m, k, s, code):
    lib = mita.load()
    assert lib.mita_workspace_bytes(ctypes.byref(sh), m, k, s) == 0
    st = lib.mita_forward(FAKE, FAKE, FAKE, m, k, s, FAKE, ctypes.byref(sh), FAKE, 1 << 40, None)
    assert st == code
    assert lib.mita_last_error().decode() != ""
    assert lib.mita_status_string(st).decode().startswith("MITA_ERR")


def test_workspace_and_pointer_checks():
    lib = mita.load()
    sh = shape()
    need = lib.mita_workspace_bytes(ctypes.byref(sh), 16, 64, 1)
    args = (16, 64, 1, FAKE, ctypes.byref(sh))
    assert lib.mita_forward(FAKE, FAKE, FAKE, *args, FAKE, need - 1, None) == mita.MITA_ERR_WORKSPACE
    assert lib.mita_forward(FAKE, FAKE, FAKE, *args, FAKE + 16, need, None) == mita.MITA_ERR_WORKSPACE
    assert lib.mita_forward(FAKE, FAKE, FAKE, *args, None, need, None) == mita.MITA_ERR_WORKSPACE
    assert lib.mita_forward(None, FAKE, FAKE, *args, FAKE, need, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_forward(FAKE + 4, FAKE, FAKE, *args, FAKE, need, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_forward(FAKE, FAKE, FAKE, 16, 64, 1, None, ctypes.byref(sh), FAKE, need, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_pool(None, 16, 64, 1, ctypes.byref(sh), FAKE, need, None, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_landmark(FAKE, None, 16, 64, 1, ctypes.byref(sh), FAKE, need, None, None, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_topk(None, 16, 64, 1, ctypes.byref(sh), FAKE, need, None, None) == mita.MITA_ERR_INVALID_ARG
    assert lib.mita_route(FAKE, 16, 64, 1, ctypes.byref(sh), FAKE, 10, None, None) == mita.MITA_ERR_WORKSPACE
    assert lib.mita_gather(FAKE, FAKE, FAKE, 16, 64, 1, FAKE, None, FAKE, need, None) == mita.MITA_ERR_INVALID_ARG


def test_status_strings():
    lib = mita.load()
    for code in (0, -1, -2, -3, -4):
        assert lib.mita_status_string(code)
    assert b"unknown" in lib.mita_status_string(42)


def test_dense_attention_argument_checks():
    # every case fails its checks before anything is enqueued (no GPU needed)
    lib = mita.load()
    good = mita.Shape(1, 2, 1000, 64, 1, 1000, 1, 16, mita.MITA_BF16)
    for sh, ptrs, code in [
        (None, (FAKE,) * 4, mita.MITA_ERR_INVALID_ARG),
        (mita.Shape(1, 2, 0, 64, 1, 1, 1, 1, mita.MITA_BF16), (FAKE,) * 4, mita.MITA_ERR_INVALID_ARG),
        (mita.Shape(1, 2, 1000, 64, 1, 1000, 1, 16, 7), (FAKE,) * 4, mita.MITA_ERR_INVALID_ARG),
        (mita.Shape(1, 2, 1000, 96, 1, 1000, 1, 16, mita.MITA_F32), (FAKE,) * 4, mita.MITA_ERR_UNSUPPORTED),
        (mita.Shape(1 << 10, 1 << 10, 1 << 12, 128, 1, 1 << 12, 1, 1, mita.MITA_F32), (FAKE,) * 4,
         mita.MITA_ERR_UNSUPPORTED),   # B H N d >= 2^31
        (good, (None, FAKE, FAKE, FAKE), mita.MITA_ERR_INVALID_ARG),
        (good, (FAKE, FAKE + 8, FAKE, FAKE), mita.MITA_ERR_INVALID_ARG),   # misaligned K
        (good, (FAKE, FAKE, FAKE, None), mita.MITA_ERR_INVALID_ARG),
    ]:
        st = lib.mita_dense_attention(*ptrs, ctypes.byref(sh) if sh is not None else None, None)
        assert st == code, (sh and (sh.N, sh.d, sh.dtype), ptrs, st)
        assert lib.mita_last_error()


def test_backward_rejects_before_launch():
    lib = mita.load()
    sh = shape(dt=mita.MITA_F32)
    assert lib.mita_backward_workspace_bytes(ctypes.byref(sh), 16, 64, 1) == 0   # bf16 only
    st = lib.mita_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 1, FAKE, FAKE, FAKE, ctypes.byref(sh), FAKE, 1 << 40,
                           FAKE, 1 << 40, None)
    assert st == mita.MITA_ERR_UNSUPPORTED
    sb = shape(dt=mita.MITA_BF16)
    n = lib.mita_backward_workspace_bytes(ctypes.byref(sb), 16, 64, 1)
    assert n > 0 and n % 256 == 0
    st = lib.mita_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 1, FAKE, FAKE, FAKE, ctypes.byref(sb), FAKE, 1 << 40,
                           None, n, None)
    assert st == mita.MITA_ERR_WORKSPACE
    st = lib.mita_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 1, FAKE, FAKE, FAKE, ctypes.byref(sb), FAKE, 1 << 40,
                           FAKE, n - 256, None)
    assert st == mita.MITA_ERR_WORKSPACE
