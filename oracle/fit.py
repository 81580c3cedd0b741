"""fp64 CPU oracle for center fitting (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like ``nanokv_oracle``: nothing in the product path
imports or calls it; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library.

The NanoKV pages store shared content in cluster centers fitted separately
for K and V (abstract; Table 5 caption: 64 centers per branch) but do not
print how they are fitted; the baseline table describes its own clustering
as K-means iterations.  This oracle takes the plainest reading: Lloyd
iterations of k-means from caller-given initial centers --

  1. assign every token to its nearest center (squared L2, ties to the lowest
     index: the encoder's own assignment);
  2. replace every center that received tokens by the mean of those tokens;
     a center that received none keeps its value;
  3. store the centers in the codec dtype (one round-half-to-even of the
     float64 mean per iteration).

Parity status: pinned by a brute-force loop version on tiny inputs, by the
closed form "one iteration from centers that reproduce the generating labels
gives the per-label means", by the empty-cluster rule and by the monotone
objective of Lloyd's method (up to storage rounding).
"""
from __future__ import annotations

import numpy as np

from . import nanokv_oracle as nk


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, one round-half-to-even.

    Works on the float64 value itself: keep 8 significant bits (the bf16
    significand) at the value's binary exponent, floored at bf16's smallest
    normal exponent so that subnormals keep their fixed quantum.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    e = np.floor(np.log2(np.abs(x[nz])))
    # guard log2 rounding at exact powers of two
    e = np.where(np.abs(x[nz]) < 2.0 ** e, e - 1, e)
    e = np.where(np.abs(x[nz]) >= 2.0 ** (e + 1), e + 1, e)
    e = np.maximum(e, -126.0)
    q = np.ldexp(1.0, (e - 7).astype(np.int64))         # bf16 quantum at this exponent
    out[nz] = np.rint(x[nz] / q) * q                     # exact: x / q has < 53 bits
    f32 = out.astype(np.float32)                          # exact: representable in bf16
    if not np.array_equal(f32.astype(np.float64), out):
        raise ValueError("bf16 rounding overflowed the float32 range")
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> the codec's storage format (bf16 bits or float32)."""
    if dtype == "bf16":
        return round_to_bf16(x64)
    return np.asarray(x64, dtype=np.float64).astype(np.float32)


def lloyd(x_stored: np.ndarray, centers_stored: np.ndarray, iters: int, dtype: str):
    """``iters`` Lloyd iterations.  Returns (centers in storage format,
    assignment of every token to the returned centers, tokens per returned
    center)."""
    x = nk.as_f64(x_stored, dtype)
    cur = np.array(centers_stored, copy=True)
    A = cur.shape[0]
    for _ in range(iters):
        mu = nk.as_f64(cur, dtype)
        idx = nk.assign(x, mu) if x.shape[0] else np.zeros(0, np.int64)
        new = mu.copy()
        for a in range(A):
            sel = idx == a
            if sel.any():
                new[a] = x[sel].sum(axis=0) / sel.sum()
        upd = np.bincount(idx, minlength=A) > 0
        stored = store(new, dtype)
        cur[upd] = stored[upd]
    mu = nk.as_f64(cur, dtype)
    idx = nk.assign(x, mu) if x.shape[0] else np.zeros(0, np.int64)
    return cur, idx.astype(np.int32), np.bincount(idx, minlength=A).astype(np.int32)


def objective(x_stored: np.ndarray, centers_stored: np.ndarray, dtype: str) -> float:
    """Sum over tokens of the squared distance to the nearest center."""
    x = nk.as_f64(x_stored, dtype)
    mu = nk.as_f64(centers_stored, dtype)
    idx = nk.assign(x, mu)
    return float(((x - mu[idx]) ** 2).sum())
