"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects malformed calls before anything reaches the GPU.

Everything here runs without a GPU: validation returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

from compressed_history_attention_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nanokv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lib.LIB_PATH),
                                reason="libnanokv.so not built")

EINVAL, EUNSUP, EWS = 1, 2, 3
FAKE = 0x1000  # non-null pointer that is never dereferenced on these paths


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = lib.load()
    names = _declared_functions()
    assert {"nkv_encode", "nkv_attend_full", "nkv_attend_fast", "nkv_lse_merge"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(lib.EXPORTS) == set(names)
    assert lib.nkv_version() == 1


def _shape(H=2, d=128, r=64, group=32, dtype=1, scale=0.0):
    return lib.nkv_shape(H, d, r, group, dtype, scale)


def _branch(A=4):
    return lib.nkv_branch(FAKE, FAKE, FAKE, FAKE, FAKE, A)


def _encode(shape, N=4, A=4, x=FAKE, ws=None, wsb=0):
    L = lib.load()
    sh = None if shape is None else ctypes.byref(shape)
    return L.nkv_encode(sh, x, N, FAKE, A, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)


def test_encode_validation():
    L = lib.load()
    assert _encode(None) == EINVAL
    assert _encode(_shape(d=100)) == EUNSUP
    assert _encode(_shape(r=48, group=32)) == EUNSUP
    assert _encode(_shape(group=12)) == EUNSUP
    assert _encode(_shape(dtype=7)) == EINVAL
    assert _encode(_shape(), A=0) == EINVAL
    assert _encode(_shape(), N=-1) == EINVAL
    assert _encode(_shape(), x=None) == EINVAL
    assert _encode(_shape(scale=float("nan"))) == EINVAL
    assert b"" != L.nkv_last_error()
    # N == 0 is a no-op that touches nothing
    assert _encode(_shape(), N=0, x=None) == 0


def _attend_fast(shape, route, r_low=16, Nq=4, N_hist=10, N_cur=2, ws=None, wsb=0, q=FAKE,
                 k=None):
    L = lib.load()
    segs, n = lib._segments(route)
    k = k or _branch()
    return L.nkv_attend_fast(ctypes.byref(shape), ctypes.byref(k), ctypes.byref(_branch()),
                             N_hist, segs, n, r_low, q, Nq, FAKE, FAKE, N_cur, FAKE, FAKE, ws,
                             wsb, None)


def test_attend_validation():
    sh = _shape()
    ok_route = [(0, 6, 1), (6, 10, 0)]
    assert _attend_fast(sh, ok_route, ws=None) == EWS           # workspace missing
    assert _attend_fast(sh, [(0, 6, 1), (5, 10, 0)]) == EINVAL  # overlap
    assert _attend_fast(sh, [(0, 6, 1)]) == EINVAL              # gap
    assert _attend_fast(sh, [(0, 6, 1), (6, 11, 0)]) == EINVAL  # out of range
    assert _attend_fast(sh, [(0, 6, 3), (6, 10, 0)]) == EINVAL  # bad mode
    assert _attend_fast(sh, ok_route, r_low=0) == EUNSUP
    assert _attend_fast(sh, ok_route, r_low=65) == EUNSUP
    assert _attend_fast(sh, ok_route, q=None) == EINVAL
    bad = _branch()
    bad.A = 0
    assert _attend_fast(sh, ok_route, k=bad) == EINVAL
    many = [(i, i + 1, i % 2) for i in range(200)]
    assert _attend_fast(sh, many, N_hist=200) == EUNSUP
    # Nq == 0 with a valid (large enough) workspace is a no-op
    need = lib.load().nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10,
                                                lib._segments(ok_route)[0], 2, 16, 0, 2)
    assert need != lib.SIZE_MAX
    assert _attend_fast(sh, ok_route, Nq=0, ws=FAKE, wsb=need) == 0


def _attend_heads(shape, widths, route=((0, 6, 1), (6, 10, 0)), Nq=4, ws=None, wsb=0):
    L = lib.load()
    segs, n = lib._segments(list(route))
    arr = None if widths is None else (ctypes.c_int32 * len(widths))(*widths)
    return L.nkv_attend_fast_heads(ctypes.byref(shape), ctypes.byref(_branch()),
                                   ctypes.byref(_branch()), 10, segs, n, arr, FAKE, Nq, FAKE,
                                   FAKE, 2, FAKE, FAKE, ws, wsb, None)


def test_attend_heads_validation():
    L = lib.load()
    sh = _shape(H=2)
    assert _attend_heads(sh, None) == EINVAL                   # no widths
    assert _attend_heads(sh, [16, 0]) == EUNSUP                # width below 1
    assert _attend_heads(sh, [16, 65]) == EUNSUP               # width above r
    assert _attend_heads(sh, [16, 32]) == EWS                  # valid, workspace missing
    assert _attend_heads(_shape(H=129, d=16, r=64, group=32), [16] * 129) == EUNSUP
    segs, n = lib._segments([(0, 6, 1), (6, 10, 0)])
    w = (ctypes.c_int32 * 2)(16, 48)
    need = L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, w, 4, 2)
    assert need != lib.SIZE_MAX and need > 0
    bad = (ctypes.c_int32 * 2)(16, 99)
    assert L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, bad, 4, 2) \
        == lib.SIZE_MAX
    # equal widths are the uniform call: the same workspace
    uni = L.nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, 48, 4, 2)
    same = (ctypes.c_int32 * 2)(48, 48)
    assert L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, same, 4, 2) == uni
    # with the same head grouping, a wider head never needs less
    narrow = (ctypes.c_int32 * 2)(16, 32)
    assert need >= L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, narrow,
                                                     4, 2)
    assert _attend_heads(sh, [16, 48], Nq=0, ws=FAKE, wsb=need) == 0


def test_attend_full_validation():
    L = lib.load()
    sh = _shape()
    k, v = _branch(), _branch()
    args = lambda N_cur, ck: (ctypes.byref(sh), ctypes.byref(k), ctypes.byref(v), 10, FAKE, 4,
                              ck, ck, N_cur, FAKE, FAKE, None, 0, None)
    assert L.nkv_attend_full(*args(3, None)) == EINVAL        # current chunk missing
    assert L.nkv_attend_full(*args(3, FAKE)) == EWS


def test_workspace_size_queries():
    L = lib.load()
    sh = _shape()
    assert L.nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10, None, 0, 0, 4, 2) > 0
    segs, n = lib._segments([(0, 6, 1), (5, 10, 0)])
    assert L.nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, 16, 4, 2) == lib.SIZE_MAX
    assert L.nkv_encode_workspace_size(ctypes.byref(_shape(d=100)), 4, 4) == lib.SIZE_MAX


def test_merge_validation():
    L = lib.load()
    assert L.nkv_lse_merge(4, 0, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == EINVAL
    assert L.nkv_lse_merge(4, 2, 16, None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == EINVAL
    assert L.nkv_lse_merge(4, 2, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 5, FAKE, None) == EINVAL
    assert L.nkv_lse_merge(0, 2, 16, None, None, None, None, None, 0, None, None) == 0


def test_status_strings():
    L = lib.load()
    assert L.nkv_status_string(0) == b"ok"
    assert L.nkv_status_string(3) == b"workspace too small"


def test_fit_validation():
    L = lib.load()
    sh = _shape()

    def call(shape=sh, x=FAKE, N=8, c=FAKE, A=4, iters=1, ws=FAKE, wsb=1 << 30):
        return L.nkv_fit_centers(None if shape is None else ctypes.byref(shape), x, N, c, A, iters,
                                 None, None, ws, wsb, None)

    assert call(shape=None) == EINVAL
    assert call(iters=-1) == EINVAL
    assert call(N=-1) == EINVAL
    assert call(A=0) == EINVAL
    assert call(A=70000) == EUNSUP
    assert call(c=None) == EINVAL
    assert call(x=None) == EINVAL
    assert call(x=FAKE + 4) == EINVAL        # x must be 16-byte aligned
    assert call(ws=None) == EWS
    assert call(wsb=16) == EWS
    assert call(shape=_shape(d=100)) == EUNSUP
    assert L.nkv_fit_workspace_size(ctypes.byref(sh), -1, 4) == lib.SIZE_MAX
    assert L.nkv_fit_workspace_size(ctypes.byref(sh), 8, 0) == lib.SIZE_MAX
    assert L.nkv_fit_workspace_size(ctypes.byref(sh), 8, 4) > 0


EHIP = 4


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="launches with fake pointers: host-only check")
@pytest.mark.parametrize("dtype,d,r", [(1, 128, 192), (0, 16, 64), (1, 64, 128)])
@pytest.mark.parametrize("route", [[(0, 10, 0)], [(0, 6, 1), (6, 10, 0)], [(0, 10, 1)],
                                   [(0, 3, 1), (3, 5, 0), (5, 10, 1)]])
@pytest.mark.parametrize("r_low", [16, 24, 48, "r"])
def test_workspace_query_matches_dispatch(dtype, d, r, route, r_low):
    """The size a call checks against is the one its dispatch lays out: with
    exactly the queried bytes the call passes every workspace check and only
    fails at its first kernel launch (no GPU here); one byte less is refused.
    Covers routes with nothing low-dimensional and widths the tuned kernels
    do not serve (r_low = 24, r_low = r), where the two once disagreed."""
    L = lib.load()
    r_low = r if r_low == "r" else r_low
    sh = _shape(H=2, d=d, r=r, group=32, dtype=dtype)
    segs, n = lib._segments(route)
    need = L.nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, r_low, 4, 2)
    assert need not in (0, lib.SIZE_MAX)
    assert _attend_fast(sh, route, r_low=r_low, ws=FAKE, wsb=need - 1) == EWS
    msg = L.nkv_last_error().decode()
    assert f"workspace of {need} bytes needed" in msg, msg
    assert _attend_fast(sh, route, r_low=r_low, ws=FAKE, wsb=need) == EHIP, L.nkv_last_error()
    # the per-head call with the same width everywhere lays out the same way
    w = (ctypes.c_int32 * 2)(r_low, r_low)
    need_h = L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, w, 4, 2)
    assert _attend_heads(sh, [r_low, r_low], route=route, ws=FAKE, wsb=need_h - 1) == EWS
    assert _attend_heads(sh, [r_low, r_low], route=route, ws=FAKE, wsb=need_h) == EHIP
    # the full read needs no more than any Fast call's all-full route
    full = L.nkv_attend_workspace_size(ctypes.byref(sh), 4, 4, 10, None, 0, 0, 4, 2)
    if route == [(0, 10, 0)]:
        assert full == need


@pytest.mark.skipif(not _no_gpu(), reason="launches with fake pointers: host-only check")
@pytest.mark.parametrize("widths", [[16, 24], [32, 48], [24, 64]])
def test_heads_workspace_query_matches_dispatch(widths):
    L = lib.load()
    sh = _shape(H=2, d=128, r=192, group=32, dtype=1)
    route = [(0, 6, 1), (6, 10, 0)]
    segs, n = lib._segments(route)
    w = (ctypes.c_int32 * 2)(*widths)
    need = L.nkv_attend_heads_workspace_size(ctypes.byref(sh), 4, 4, 10, segs, n, w, 4, 2)
    assert _attend_heads(sh, widths, route=route, ws=FAKE, wsb=need - 1) == EWS
    assert _attend_heads(sh, widths, route=route, ws=FAKE, wsb=need) == EHIP


def test_merge_aliasing_rules():
    """Only exact aliasing is accepted: an fp32 output that is a part's own
    array, an LSE output that is a part's own LSE array."""
    L = lib.load()
    Nq, H, d = 4, 2, 8
    ob = Nq * H * d * 4
    lb = Nq * H * 4
    base = 0x100000
    oa, ob_, la, lb_ = base, base + 4 * ob, base + 8 * ob, base + 8 * ob + 4096
    out, lout = base + 12 * ob, base + 16 * ob

    def call(o=out, lo=lout, dt=0):
        return L.nkv_lse_merge(Nq, H, d, oa, la, ob_, lb_, o, dt, lo, None)

    # bf16 output over a part's bytes races
    assert call(o=oa, dt=1) == EINVAL
    # a shifted view of a part
    assert call(o=oa + 16) == EINVAL
    assert call(lo=la + 4) == EINVAL
    # output over an LSE array
    assert call(o=la) == EINVAL
    # d not a multiple of 4 is accepted (scalar path): validation passes and
    # only the launch fails without a GPU
    if _no_gpu():
        assert L.nkv_lse_merge(Nq, H, 6, oa, la, ob_, lb_, out, 0, lout, None) == EHIP
        assert call(o=oa, lo=la) == EHIP          # exact fp32 aliasing
        assert call(o=ob_, lo=lb_) == EHIP
