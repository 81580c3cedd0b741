"""ctypes binding of libnanokv (argument marshalling only).

The functions named like the C entry points (``nkv_encode``,
``nkv_attend_full``, ``nkv_attend_fast``, ``nkv_lse_merge`` and the
workspace-size queries) take torch tensors that already live on the GPU,
pass their device pointers and the current HIP stream to the library and
raise ``NkvError`` on a non-zero status.  The helpers ``encode``,
``attend_full``, ``attend_fast`` and ``lse_merge`` additionally allocate the
outputs and the workspace with torch.  No computation happens here: every
step runs in the HIP kernels of ``libnanokv.so``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnanokv.so")

NKV_F32, NKV_BF16 = 0, 1
NKV_FULL, NKV_LOW = 0, 1
MAX_SEGMENTS = 64
SIZE_MAX = ctypes.c_size_t(-1).value
_DT = {"f32": NKV_F32, "bf16": NKV_BF16}
_TORCH_DT = {NKV_F32: torch.float32, NKV_BF16: torch.bfloat16}


class NkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libnanokv status {status}: {msg}")
        self.status = status


class nkv_shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("r", ctypes.c_int32),
                ("group", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class nkv_branch(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("centers", ctypes.c_void_p),
                ("decoder", ctypes.c_void_p), ("A", ctypes.c_int32)]


class nkv_segment(ctypes.Structure):
    _fields_ = [("begin", ctypes.c_int64), ("end", ctypes.c_int64), ("mode", ctypes.c_int32)]


class nkv_low_maps(ctypes.Structure):
    _fields_ = [("q_map", ctypes.c_void_p), ("o_map", ctypes.c_void_p), ("ld", ctypes.c_int32)]


class nkv_route_policy(ctypes.Structure):
    _fields_ = [("frame_tokens", ctypes.c_int64), ("recent_frames", ctypes.c_int32),
                ("sink_frames", ctypes.c_int32), ("anchor_every", ctypes.c_int32),
                ("all_full_frames", ctypes.c_int32), ("layer_full", ctypes.c_int32)]


class nkv_storage(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("idx", "codes", "scales", "cached", "centers",
                                               "encoders", "decoders", "resident", "total",
                                               "original")] + \
               [(n, ctypes.c_double) for n in ("cr_effective", "cr_cached", "cr_nominal")]


class nkv_cache_branch(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("centers", ctypes.c_void_p),
                ("encoder", ctypes.c_void_p), ("decoder", ctypes.c_void_p),
                ("A", ctypes.c_int32)]


class nkv_layer_cache(ctypes.Structure):
    _fields_ = [("k", nkv_cache_branch), ("v", nkv_cache_branch),
                ("n_hist", ctypes.c_int64), ("capacity", ctypes.c_int64)]


class nkv_prof_entry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("ms", ctypes.c_double), ("count", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libnanokv.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "compressed_history_attention_amd/build.py (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH, BR, SG = ctypes.POINTER(nkv_shape), ctypes.POINTER(nkv_branch), ctypes.POINTER(nkv_segment)
    LC, RP = ctypes.POINTER(nkv_layer_cache), ctypes.POINTER(nkv_route_policy)
    MP = ctypes.POINTER(nkv_low_maps)
    sig = {
        "nkv_version": (ctypes.c_int, []),
        "nkv_last_error": (ctypes.c_char_p, []),
        "nkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "nkv_force_generic": (None, [ctypes.c_int]),
        "nkv_encode_workspace_size": (SZ, [SH, I64, I32]),
        "nkv_encode": (ctypes.c_int, [SH, P, I64, P, I32, P, P, P, P, P, SZ, P]),
        "nkv_encode_noalloc": (ctypes.c_int, [SH, P, I64, P, I32, P, P, P, P, P]),
        "nkv_attend_workspace_size": (SZ, [SH, I32, I32, I64, SG, I32, I32, I64, I64]),
        "nkv_attend_full": (ctypes.c_int, [SH, BR, BR, I64, P, I64, P, P, I64, P, P, P, SZ, P]),
        "nkv_attend_fast": (ctypes.c_int, [SH, BR, BR, I64, SG, I32, I32, P, I64, P, P, I64, P,
                                           P, P, SZ, P]),
        "nkv_attend_heads_workspace_size": (SZ, [SH, I32, I32, I64, SG, I32, ctypes.POINTER(I32),
                                                 I64, I64]),
        "nkv_attend_fast_heads": (ctypes.c_int, [SH, BR, BR, I64, SG, I32, ctypes.POINTER(I32), P,
                                                 I64, P, P, I64, P, P, P, SZ, P]),
        "nkv_attend_maps_workspace_size": (SZ, [SH, I32, I32, I64, SG, I32, ctypes.POINTER(I32),
                                                MP, I64, I64]),
        "nkv_attend_fast_maps": (ctypes.c_int, [SH, BR, BR, I64, SG, I32, ctypes.POINTER(I32), MP,
                                                P, I64, P, P, I64, P, P, P, SZ, P]),
        "nkv_lse_merge": (ctypes.c_int, [I64, I32, I32, P, P, P, P, P, I32, P, P]),
        "nkv_fit_workspace_size": (SZ, [SH, I64, I32]),
        "nkv_fit_centers": (ctypes.c_int, [SH, P, I64, P, I32, I32, P, P, P, SZ, P]),
        "nkv_route_segments": (ctypes.c_int, [ctypes.POINTER(nkv_route_policy), I64, SG, I32,
                                              ctypes.POINTER(I32)]),
        "nkv_storage_account": (ctypes.c_int, [SH, I32, I32, I64, ctypes.POINTER(nkv_storage)]),
        "nkv_layer_attend_workspace_size": (SZ, [SH, LC, RP, ctypes.POINTER(I32), I64, I64]),
        "nkv_layer_attend": (ctypes.c_int, [SH, LC, RP, ctypes.POINTER(I32), P, I64, P, P, I64,
                                            P, P, P, SZ, P]),
        "nkv_layer_append_workspace_size": (SZ, [SH, LC, I64]),
        "nkv_layer_append": (ctypes.c_int, [SH, LC, P, P, I64, P, SZ, P]),
        "nkv_profile_enable": (None, [ctypes.c_int]),
        "nkv_profile_read": (ctypes.c_int, [ctypes.POINTER(nkv_prof_entry), I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTS = ("nkv_version", "nkv_last_error", "nkv_status_string", "nkv_force_generic",
           "nkv_encode_workspace_size", "nkv_encode", "nkv_attend_workspace_size",
           "nkv_attend_full", "nkv_attend_fast", "nkv_attend_heads_workspace_size",
           "nkv_attend_fast_heads", "nkv_attend_maps_workspace_size", "nkv_attend_fast_maps",
           "nkv_lse_merge", "nkv_fit_workspace_size", "nkv_fit_centers", "nkv_route_segments", "nkv_storage_account",
           "nkv_layer_attend_workspace_size", "nkv_layer_attend", "nkv_layer_append_workspace_size",
           "nkv_layer_append", "nkv_profile_enable", "nkv_profile_read", "nkv_encode_noalloc")

NOALLOC_SCRATCH_BYTES = 32 << 20  # NKV_NOALLOC_SCRATCH_BYTES


def _check(status: int):
    if status != 0:
        raise NkvError(status, load().nkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libnanokv must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ----------------------------------------------------------------------------
# Python-side descriptions
# ----------------------------------------------------------------------------

@dataclass
class Shape:
    H: int
    d: int
    r: int
    group: int
    dtype: str = "bf16"
    softmax_scale: float = 0.0

    def c(self) -> nkv_shape:
        return nkv_shape(self.H, self.d, self.r, self.group, _DT[self.dtype], self.softmax_scale)

    @property
    def W(self) -> int:
        return self.H * self.d

    @property
    def torch_dtype(self):
        return _TORCH_DT[_DT[self.dtype]]


@dataclass
class Branch:
    """Compressed history of one branch on the GPU (idx, codes, scales) plus
    its centers [A, W] and decoder [W, r]."""
    idx: torch.Tensor
    codes: torch.Tensor
    scales: torch.Tensor
    centers: torch.Tensor
    decoder: torch.Tensor

    def c(self) -> nkv_branch:
        return nkv_branch(_ptr(self.idx), _ptr(self.codes), _ptr(self.scales), _ptr(self.centers),
                          _ptr(self.decoder), int(self.centers.shape[0]))

    @property
    def A(self) -> int:
        return int(self.centers.shape[0])


def _segments(route: Optional[Sequence[Tuple[int, int, int]]]):
    if not route:
        return None, 0
    arr = (nkv_segment * len(route))(*[nkv_segment(int(b), int(e), int(m)) for b, e, m in route])
    return arr, len(route)


# ----------------------------------------------------------------------------
# entry points with the C names
# ----------------------------------------------------------------------------

def nkv_version() -> int:
    return load().nkv_version()


def nkv_force_generic(on: bool) -> None:
    load().nkv_force_generic(1 if on else 0)


def nkv_profile_enable(on: bool) -> None:
    load().nkv_profile_enable(1 if on else 0)


def nkv_profile_read(max_entries: int = 64) -> dict:
    """{stage: (total ms, launches)} recorded since the last read."""
    buf = (nkv_prof_entry * max_entries)()
    n = load().nkv_profile_read(buf, max_entries)
    if n < 0:
        raise NkvError(4, "profile read failed")
    return {buf[i].name.decode(): (buf[i].ms, buf[i].count) for i in range(n)}


def nkv_encode_workspace_size(shape: Shape, N: int, A: int) -> int:
    n = load().nkv_encode_workspace_size(ctypes.byref(shape.c()), N, A)
    if n == SIZE_MAX:
        raise NkvError(1, "invalid encode shape")
    return n


def nkv_encode(shape: Shape, x, centers, encoder, idx, codes, scales, ws=None, stream=None):
    N = int(x.shape[0]) if x is not None else 0
    _check(load().nkv_encode(ctypes.byref(shape.c()), _ptr(x), N, _ptr(centers),
                             int(centers.shape[0]), _ptr(encoder), _ptr(idx), _ptr(codes),
                             _ptr(scales), _ptr(ws), 0 if ws is None else ws.numel(),
                             _stream(stream)))


def nkv_encode_noalloc(shape: Shape, x, centers, encoder, idx, codes, scales, stream=None):
    """nkv_encode with the library's fixed device scratch: no workspace."""
    N = int(x.shape[0]) if x is not None else 0
    _check(load().nkv_encode_noalloc(ctypes.byref(shape.c()), _ptr(x), N, _ptr(centers),
                                     int(centers.shape[0]), _ptr(encoder), _ptr(idx), _ptr(codes),
                                     _ptr(scales), _stream(stream)))


def nkv_attend_workspace_size(shape: Shape, A_k: int, A_v: int, N_hist: int, route, r_low: int,
                              Nq: int, N_cur: int) -> int:
    segs, n = _segments(route)
    res = load().nkv_attend_workspace_size(ctypes.byref(shape.c()), A_k, A_v, N_hist, segs, n,
                                           r_low, Nq, N_cur)
    if res == SIZE_MAX:
        raise NkvError(1, load().nkv_last_error().decode() or "invalid attend arguments")
    return res


def _widths(shape: Shape, r_low_h):
    arr = (ctypes.c_int32 * shape.H)(*[int(x) for x in r_low_h])
    if len(r_low_h) != shape.H:
        raise ValueError(f"need {shape.H} per-head widths, got {len(r_low_h)}")
    return arr


def nkv_attend_heads_workspace_size(shape: Shape, A_k: int, A_v: int, N_hist: int, route,
                                    r_low_h, Nq: int, N_cur: int) -> int:
    segs, n = _segments(route)
    res = load().nkv_attend_heads_workspace_size(ctypes.byref(shape.c()), A_k, A_v, N_hist, segs,
                                                 n, _widths(shape, r_low_h), Nq, N_cur)
    if res == SIZE_MAX:
        raise NkvError(1, load().nkv_last_error().decode() or "invalid attend arguments")
    return res


def nkv_attend_fast_heads(shape: Shape, k: Branch, v: Branch, N_hist: int, route, r_low_h, q,
                          cur_k, cur_v, out, lse, ws=None, stream=None):
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    segs, n = _segments(route)
    _check(load().nkv_attend_fast_heads(ctypes.byref(shape.c()), ctypes.byref(k.c()),
                                        ctypes.byref(v.c()), N_hist, segs, n,
                                        _widths(shape, r_low_h), _ptr(q), int(q.shape[0]),
                                        _ptr(cur_k), _ptr(cur_v), N_cur, _ptr(out), _ptr(lse),
                                        _ptr(ws), 0 if ws is None else ws.numel(),
                                        _stream(stream)))


def _maps(q_map, o_map) -> nkv_low_maps:
    if q_map.shape != o_map.shape or q_map.dim() != 2:
        raise ValueError("q_map and o_map must both be [W, ld]")
    return nkv_low_maps(_ptr(q_map), _ptr(o_map), int(q_map.shape[1]))


def nkv_attend_maps_workspace_size(shape: Shape, A_k: int, A_v: int, N_hist: int, route, r_low_h,
                                   q_map, o_map, Nq: int, N_cur: int) -> int:
    segs, n = _segments(route)
    res = load().nkv_attend_maps_workspace_size(ctypes.byref(shape.c()), A_k, A_v, N_hist, segs,
                                                n, _widths(shape, r_low_h),
                                                ctypes.byref(_maps(q_map, o_map)), Nq, N_cur)
    if res == SIZE_MAX:
        raise NkvError(1, load().nkv_last_error().decode() or "invalid attend arguments")
    return res


def nkv_attend_fast_maps(shape: Shape, k: Branch, v: Branch, N_hist: int, route, r_low_h, q_map,
                         o_map, q, cur_k, cur_v, out, lse, ws=None, stream=None):
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    segs, n = _segments(route)
    _check(load().nkv_attend_fast_maps(ctypes.byref(shape.c()), ctypes.byref(k.c()),
                                       ctypes.byref(v.c()), N_hist, segs, n,
                                       _widths(shape, r_low_h),
                                       ctypes.byref(_maps(q_map, o_map)), _ptr(q),
                                       int(q.shape[0]), _ptr(cur_k), _ptr(cur_v), N_cur,
                                       _ptr(out), _ptr(lse), _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(stream)))


def nkv_attend_full(shape: Shape, k: Branch, v: Branch, N_hist: int, q, cur_k, cur_v, out, lse,
                    ws=None, stream=None):
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    _check(load().nkv_attend_full(ctypes.byref(shape.c()), ctypes.byref(k.c()),
                                  ctypes.byref(v.c()), N_hist, _ptr(q), int(q.shape[0]),
                                  _ptr(cur_k), _ptr(cur_v), N_cur, _ptr(out), _ptr(lse),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def nkv_attend_fast(shape: Shape, k: Branch, v: Branch, N_hist: int, route, r_low: int, q, cur_k,
                    cur_v, out, lse, ws=None, stream=None):
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    segs, n = _segments(route)
    _check(load().nkv_attend_fast(ctypes.byref(shape.c()), ctypes.byref(k.c()),
                                  ctypes.byref(v.c()), N_hist, segs, n, r_low, _ptr(q),
                                  int(q.shape[0]), _ptr(cur_k), _ptr(cur_v), N_cur, _ptr(out),
                                  _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream)))


def nkv_lse_merge(H: int, d: int, o_a, lse_a, o_b, lse_b, out, lse_out, stream=None):
    dt = NKV_F32 if out.dtype == torch.float32 else NKV_BF16
    _check(load().nkv_lse_merge(int(o_a.shape[0]), H, d, _ptr(o_a), _ptr(lse_a), _ptr(o_b),
                                _ptr(lse_b), _ptr(out), dt, _ptr(lse_out), _stream(stream)))


def nkv_fit_workspace_size(shape: Shape, N: int, A: int) -> int:
    n = load().nkv_fit_workspace_size(ctypes.byref(shape.c()), N, A)
    if n == SIZE_MAX:
        raise NkvError(1, "invalid fit arguments")
    return n


def nkv_fit_centers(shape: Shape, x, centers, iters: int, idx=None, counts=None, ws=None,
                    stream=None):
    N = int(x.shape[0])
    _check(load().nkv_fit_centers(ctypes.byref(shape.c()), _ptr(x), N, _ptr(centers),
                                  int(centers.shape[0]), int(iters), _ptr(idx), _ptr(counts),
                                  _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def fit_centers(shape: Shape, x, centers, iters: int, stream=None):
    """Lloyd iterations in place on ``centers``; returns (centers, idx, counts)
    with idx/counts the assignment to the returned centers."""
    N, A = int(x.shape[0]), int(centers.shape[0])
    idx = torch.empty(N, dtype=torch.int32, device=centers.device)
    counts = torch.empty(A, dtype=torch.int32, device=centers.device)
    ws = _workspace(nkv_fit_workspace_size(shape, N, A), centers.device)
    nkv_fit_centers(shape, x, centers, iters, idx if N else None, counts, ws=ws, stream=stream)
    _keep(stream, ws, idx, counts)
    return centers, idx, counts


@dataclass(frozen=True)
class RoutePolicy:
    """Per-layer full-dimensional routing policy (mirrors nkv_route_policy)."""
    frame_tokens: int
    recent_frames: int = 0
    sink_frames: int = 0
    anchor_every: int = 0
    all_full_frames: int = 0
    layer_full: bool = False

    def c(self) -> nkv_route_policy:
        return nkv_route_policy(int(self.frame_tokens), int(self.recent_frames),
                                int(self.sink_frames), int(self.anchor_every),
                                int(self.all_full_frames), 1 if self.layer_full else 0)


def nkv_route_segments(policy: RoutePolicy, n_hist: int):
    """[(begin, end, mode)] of the policy over n_hist history tokens."""
    L, pol, n = load(), policy.c(), ctypes.c_int32(0)
    st = L.nkv_route_segments(ctypes.byref(pol), n_hist, None, 0, ctypes.byref(n))
    if st != 0 and n.value == 0 and n_hist > 0:
        _check(st)
    buf = (nkv_segment * max(1, n.value))()
    _check(L.nkv_route_segments(ctypes.byref(pol), n_hist, buf, n.value, ctypes.byref(n)))
    return [(buf[i].begin, buf[i].end, buf[i].mode) for i in range(n.value)]


def nkv_storage_account(shape: Shape, A_k: int, A_v: int, n_hist: int) -> dict:
    out = nkv_storage()
    _check(load().nkv_storage_account(ctypes.byref(shape.c()), A_k, A_v, n_hist,
                                      ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in nkv_storage._fields_}


class LayerCache:
    """One layer's compressed history on the GPU (both branches) with room
    for ``capacity`` tokens, plus the layer's codecs.  ``n_hist`` lives in
    the C descriptor that nkv_layer_append advances."""

    def __init__(self, shape: Shape, capacity: int, centers, encoders, decoders, device):
        self.shape = shape
        dev = torch.device(device)
        self.codec = (tuple(centers), tuple(encoders), tuple(decoders))
        self.idx = [torch.empty(capacity, dtype=torch.int32, device=dev) for _ in range(2)]
        self.codes = [torch.empty((capacity, shape.r // 2), dtype=torch.uint8, device=dev)
                      for _ in range(2)]
        self.scales = [torch.empty((capacity, shape.r // shape.group), dtype=torch.int16,
                                   device=dev) for _ in range(2)]
        br = [nkv_cache_branch(_ptr(self.idx[b]), _ptr(self.codes[b]), _ptr(self.scales[b]),
                               _ptr(centers[b]), _ptr(encoders[b]), _ptr(decoders[b]),
                               int(centers[b].shape[0])) for b in range(2)]
        self.desc = nkv_layer_cache(br[0], br[1], 0, int(capacity))

    @property
    def n_hist(self) -> int:
        return int(self.desc.n_hist)

    @property
    def capacity(self) -> int:
        return int(self.desc.capacity)

    def branch(self, b: int) -> Branch:
        """The stored history of branch b (0 = K, 1 = V) as a Branch view."""
        n = self.n_hist
        return Branch(self.idx[b][:n], self.codes[b][:n], self.scales[b][:n],
                      self.codec[0][b], self.codec[2][b])

    def history_bytes(self) -> int:
        """Bytes of the stored records (both branches) at the current length."""
        n = self.n_hist
        return sum(t[:n].numel() * t.element_size()
                   for t in (*self.idx, *self.codes, *self.scales))


def nkv_layer_attend_workspace_size(shape: Shape, cache: LayerCache, policy: RoutePolicy,
                                    r_low_h, Nq: int, N_cur: int) -> int:
    w = None if r_low_h is None else _widths(shape, r_low_h)
    res = load().nkv_layer_attend_workspace_size(ctypes.byref(shape.c()),
                                                 ctypes.byref(cache.desc),
                                                 ctypes.byref(policy.c()), w, Nq, N_cur)
    if res == SIZE_MAX:
        raise NkvError(1, load().nkv_last_error().decode() or "invalid layer attend arguments")
    return res


def nkv_layer_attend(shape: Shape, cache: LayerCache, policy: RoutePolicy, r_low_h, q, cur_k,
                     cur_v, out, lse, ws=None, stream=None):
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    w = None if r_low_h is None else _widths(shape, r_low_h)
    _check(load().nkv_layer_attend(ctypes.byref(shape.c()), ctypes.byref(cache.desc),
                                   ctypes.byref(policy.c()), w, _ptr(q), int(q.shape[0]),
                                   _ptr(cur_k), _ptr(cur_v), N_cur, _ptr(out), _ptr(lse),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def nkv_layer_append_workspace_size(shape: Shape, cache: LayerCache, N: int) -> int:
    res = load().nkv_layer_append_workspace_size(ctypes.byref(shape.c()),
                                                 ctypes.byref(cache.desc), N)
    if res == SIZE_MAX:
        raise NkvError(1, load().nkv_last_error().decode() or "invalid append arguments")
    return res


def nkv_layer_append(shape: Shape, cache: LayerCache, k_new, v_new, ws=None, stream=None):
    N = int(k_new.shape[0])
    if int(v_new.shape[0]) != N:
        raise ValueError("k_new and v_new need the same number of rows")
    _check(load().nkv_layer_append(ctypes.byref(shape.c()), ctypes.byref(cache.desc),
                                   _ptr(k_new), _ptr(v_new), N, _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)))


# ----------------------------------------------------------------------------
# allocating helpers
# ----------------------------------------------------------------------------

def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def _keep(stream, *tensors) -> None:
    """Tensors allocated here come from torch's caching allocator on the
    current stream.  When the kernels run on another ``stream``, mark them
    used there, so that their memory is not handed out again before that
    stream's work is done (the workspace is freed as soon as we return)."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def encode(shape: Shape, x, centers, encoder, out=None, stream=None):
    """Encode tokens x [N, W]; returns (idx int32 [N], codes uint8 [N, r/2],
    scales int16 [N, r/group] holding fp16 bits).  ``out`` may supply the
    three output tensors (e.g. views into a preallocated history)."""
    N = int(x.shape[0])
    dev = x.device
    if out is None:
        out = (torch.empty(N, dtype=torch.int32, device=dev),
               torch.empty((N, shape.r // 2), dtype=torch.uint8, device=dev),
               torch.empty((N, shape.r // shape.group), dtype=torch.int16, device=dev))
    ws = _workspace(nkv_encode_workspace_size(shape, N, int(centers.shape[0])), dev)
    nkv_encode(shape, x, centers, encoder, *out, ws=ws, stream=stream)
    _keep(stream, ws, *out)
    return out


def attend_full(shape: Shape, k: Branch, v: Branch, N_hist: int, q, cur_k=None, cur_v=None,
                ws=None, stream=None):
    Nq = int(q.shape[0])
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    out = torch.empty((Nq, shape.W), dtype=shape.torch_dtype, device=q.device)
    lse = torch.empty((Nq, shape.H), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = _workspace(nkv_attend_workspace_size(shape, k.A, v.A, N_hist, None, 0, Nq, N_cur),
                        q.device)
    nkv_attend_full(shape, k, v, N_hist, q, cur_k, cur_v, out, lse, ws=ws, stream=stream)
    _keep(stream, ws, out, lse)
    return out, lse


def attend_fast(shape: Shape, k: Branch, v: Branch, N_hist: int, route, r_low, q,
                cur_k=None, cur_v=None, ws=None, stream=None, maps=None):
    """r_low: one width for every head, or a sequence of one width per head
    (nkv_attend_fast_heads).  maps: optional (q_map, o_map), both [W, ld],
    replacing the decoders in the query reduction and output restoration
    (nkv_attend_fast_maps)."""
    Nq = int(q.shape[0])
    N_cur = 0 if cur_k is None else int(cur_k.shape[0])
    out = torch.empty((Nq, shape.W), dtype=shape.torch_dtype, device=q.device)
    lse = torch.empty((Nq, shape.H), dtype=torch.float32, device=q.device)
    if maps is not None:
        widths = [int(r_low)] * shape.H if isinstance(r_low, (int, np.integer)) else r_low
        if ws is None:
            ws = _workspace(nkv_attend_maps_workspace_size(shape, k.A, v.A, N_hist, route, widths,
                                                           maps[0], maps[1], Nq, N_cur), q.device)
        nkv_attend_fast_maps(shape, k, v, N_hist, route, widths, maps[0], maps[1], q, cur_k, cur_v,
                             out, lse, ws=ws, stream=stream)
        _keep(stream, ws, out, lse)
        return out, lse
    if not isinstance(r_low, (int, np.integer)):
        if ws is None:
            ws = _workspace(nkv_attend_heads_workspace_size(shape, k.A, v.A, N_hist, route, r_low,
                                                            Nq, N_cur), q.device)
        nkv_attend_fast_heads(shape, k, v, N_hist, route, r_low, q, cur_k, cur_v, out, lse,
                              ws=ws, stream=stream)
        _keep(stream, ws, out, lse)
        return out, lse
    if ws is None:
        ws = _workspace(nkv_attend_workspace_size(shape, k.A, v.A, N_hist, route, r_low, Nq,
                                                  N_cur), q.device)
    nkv_attend_fast(shape, k, v, N_hist, route, r_low, q, cur_k, cur_v, out, lse, ws=ws,
                    stream=stream)
    _keep(stream, ws, out, lse)
    return out, lse


def lse_merge(H: int, d: int, o_a, lse_a, o_b, lse_b, out_dtype=torch.float32, stream=None):
    out = torch.empty(o_a.shape, dtype=out_dtype, device=o_a.device)
    lse = torch.empty(lse_a.shape, dtype=torch.float32, device=o_a.device)
    nkv_lse_merge(H, d, o_a, lse_a, o_b, lse_b, out, lse, stream=stream)
    _keep(stream, out, lse)
    return out, lse
