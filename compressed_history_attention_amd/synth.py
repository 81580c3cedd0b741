"""Seeded synthetic workloads for compressed-history attention.

This module only *draws* inputs; it holds none of the method's arithmetic (no
center assignment, projection, quantisation, decoding or attention).  Both the
GPU path and the fp64 oracle consume the exact bits it produces.

Workload shapes follow the video backbones the NanoKV pages describe
(NanoKV: High-Ratio KV Cache Compression for Autoregressive Video Generation,
Table 9: head dimension 128; Table 5: per-branch rank and shared centers).
History tokens are drawn as ``x = mu[a] + U z`` with ``a`` uniform over the
centers, ``U`` a random orthonormal ``W x r`` basis and
``z_i ~ N(0, 1/(i+1))`` (a decaying spectrum), computed in float64 and rounded
once, round-half-to-even, to the storage dtype.  Decoders are random
orthonormal ``W x r`` matrices (seeded QR) rounded to the storage dtype and the
encoder is exactly the transpose of the rounded decoder.

Storage conventions (shared with the C ABI):
  * ``f32`` tensors are ``np.float32`` arrays;
  * ``bf16`` tensors are ``np.uint16`` arrays holding bfloat16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

CHUNK = 4680  # tokens per latent chunk in the video workloads

# RNG stream ids: every tensor has its own stream keyed by (seed, id, part)
_S_CENTERS = (0, 1)      # K, V centers
_S_BASIS = (2, 3)        # generating bases U_K, U_V
_S_ASSIGN = (4, 5)       # history center labels K, V
_S_COEF = (6, 7)         # history latent coefficients K, V
_S_DECODER = (8, 9)      # decoders D_K, D_V
_S_QUERY = 10
_S_CUR_ASSIGN = (11, 12)
_S_CUR_COEF = (13, 14)
_S_NEW_ASSIGN = (15, 16)
_S_NEW_COEF = (17, 18)


@dataclass(frozen=True)
class Config:
    name: str
    H: int
    d: int
    r: int
    A: int
    group: int
    n_hist: int          # history tokens already in the cache
    Nq: int
    N_cur: int
    dtype: str           # "f32" | "bf16"
    seed: int
    mode: str            # "full" | "fast"
    r_low: int = 0
    n_full_tail: int = 0  # most recent history tokens routed full-dimensional
    n_new: int = 0        # tokens encoded and appended before attending
    center_scale: float = 1.0  # multiplies the centers (test-only variants)
    chunk: int = CHUNK

    @property
    def W(self) -> int:
        return self.H * self.d

    @property
    def n_attend(self) -> int:
        """History length seen by attention (existing + appended)."""
        return self.n_hist + self.n_new

    @property
    def tau(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def segments(self) -> List[Tuple[int, int, int]]:
        """Routing policy as (begin, end, mode) with mode 0 = full, 1 = low.

        Oldest tokens come first; the most recent ``n_full_tail`` tokens are
        read full-dimensionally, everything older low-dimensionally.
        """
        n = self.n_attend
        if self.mode == "full":
            return [(0, n, 0)] if n else []
        split = max(0, n - self.n_full_tail)
        segs = []
        if split > 0:
            segs.append((0, split, 1))
        if n - split > 0:
            segs.append((split, n, 0))
        return segs


CONFIGS: Dict[str, Config] = {
    # tiny fp32 case: full path only
    "C0": Config("C0", H=2, d=16, r=8, A=4, group=8, n_hist=64, Nq=16, N_cur=16,
                 dtype="f32", seed=0, mode="full", chunk=64),
    # Wan-1.3B-like layer, full-dimensional path
    "C1": Config("C1", H=12, d=128, r=192, A=256, group=32, n_hist=4 * CHUNK,
                 Nq=CHUNK, N_cur=CHUNK, dtype="bf16", seed=1, mode="full"),
    # same tensors through the mixed-dimensional path
    "C2": Config("C2", H=12, d=128, r=192, A=256, group=32, n_hist=4 * CHUNK,
                 Nq=CHUNK, N_cur=CHUNK, dtype="bf16", seed=1, mode="fast",
                 r_low=48, n_full_tail=CHUNK),
    # larger backbone layer, mixed-dimensional
    "C3": Config("C3", H=24, d=128, r=384, A=1024, group=32, n_hist=12 * CHUNK,
                 Nq=CHUNK, N_cur=CHUNK, dtype="bf16", seed=3, mode="fast",
                 r_low=96, n_full_tail=2 * CHUNK),
    # long rollout: encode one new chunk, append to 32 chunks, attend 33
    "C4": Config("C4", H=24, d=128, r=384, A=1024, group=32, n_hist=32 * CHUNK,
                 Nq=CHUNK, N_cur=CHUNK, dtype="bf16", seed=4, mode="fast",
                 r_low=96, n_full_tail=4 * CHUNK, n_new=CHUNK),
}


def small_config(base: str = "C3", **kw) -> Config:
    """A reduced copy of a workload for parity tests (several tiles + tails)."""
    return replace(CONFIGS[base], **kw)


# ----------------------------------------------------------------------------
# storage rounding (integer round-half-to-even), no method arithmetic
# ----------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once, half-to-even, to bfloat16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in generated data")
    b = x.view(np.uint64).copy()
    # bfloat16 keeps 7 of the 52 fraction bits: drop 45 with round-half-even
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    b = b + (np.uint64((1 << 44) - 1) + lsb)
    b &= ~np.uint64((1 << 45) - 1)
    y = b.view(np.float64)
    a = np.abs(y)
    if np.any((a != 0) & ((a < 2.0 ** -126) | (a >= 2.0 ** 128))):
        raise ValueError("generated value outside the bfloat16 normal range")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    raise ValueError(dtype)


def load64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor (used by the generator itself)."""
    if dtype == "f32":
        return a.astype(np.float64)
    return bf16_bits_to_f64(a)


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([seed, *ids])


def _orthonormal(rng: np.random.Generator, W: int, r: int) -> np.ndarray:
    g = rng.standard_normal((W, r))
    q, _ = np.linalg.qr(g)
    return q


@dataclass
class Workload:
    """Lazily generated tensors of one configuration."""
    cfg: Config
    _cache: dict = field(default_factory=dict)

    def _memo(self, key, fn):
        if key not in self._cache:
            self._cache[key] = fn()
        return self._cache[key]

    # codec parameters -----------------------------------------------------
    def centers(self, b: int) -> np.ndarray:
        c = self.cfg

        def make():
            g = _rng(c.seed, _S_CENTERS[b]).standard_normal((c.A, c.W))
            return store(g * c.center_scale, c.dtype)
        return self._memo(("centers", b), make)

    def basis(self, b: int) -> np.ndarray:
        c = self.cfg
        return self._memo(("basis", b),
                          lambda: _orthonormal(_rng(c.seed, _S_BASIS[b]), c.W, c.r))

    def decoder(self, b: int) -> np.ndarray:
        """D [W, r] in storage dtype."""
        c = self.cfg
        return self._memo(("decoder", b), lambda: store(
            _orthonormal(_rng(c.seed, _S_DECODER[b]), c.W, c.r), c.dtype))

    def encoder(self, b: int) -> np.ndarray:
        """E = D^T [r, W], the exact transpose of the stored decoder."""
        return self._memo(("encoder", b),
                          lambda: np.ascontiguousarray(self.decoder(b).T))

    # tokens ---------------------------------------------------------------
    def _tokens(self, b: int, n: int, s_assign: int, s_coef: int, part: int):
        c = self.cfg
        a = _rng(c.seed, s_assign, part).integers(0, c.A, size=n)
        sd = np.sqrt(1.0 / (np.arange(c.r) + 1.0))
        z = _rng(c.seed, s_coef, part).standard_normal((n, c.r)) * sd
        mu = load64(self.centers(b), c.dtype)
        x = mu[a] + z @ self.basis(b).T
        return store(x, c.dtype), a.astype(np.int32), z

    def history_chunk(self, b: int, k: int):
        """Chunk ``k`` of the existing history: (tokens, labels, latent z)."""
        c = self.cfg
        lo = k * c.chunk
        n = min(c.chunk, c.n_hist - lo)
        if n <= 0:
            raise IndexError(k)
        return self._tokens(b, n, _S_ASSIGN[b], _S_COEF[b], k)

    def n_history_chunks(self) -> int:
        c = self.cfg
        return (c.n_hist + c.chunk - 1) // c.chunk

    def history_tokens(self, b: int) -> np.ndarray:
        parts = [self.history_chunk(b, k)[0] for k in range(self.n_history_chunks())]
        if not parts:
            return np.zeros((0, self.cfg.W), dtype=np.float32 if self.cfg.dtype == "f32" else np.uint16)
        return np.concatenate(parts, axis=0)

    def current(self, b: int) -> np.ndarray:
        """Uncompressed current-chunk K or V [N_cur, W]."""
        c = self.cfg
        return self._memo(("cur", b), lambda: self._tokens(
            b, c.N_cur, _S_CUR_ASSIGN[b], _S_CUR_COEF[b], 0)[0])

    def new_chunk(self, b: int):
        """Tokens encoded and appended before attending: (tokens, labels, z)."""
        c = self.cfg
        return self._memo(("new", b), lambda: self._tokens(
            b, c.n_new, _S_NEW_ASSIGN[b], _S_NEW_COEF[b], 0))

    def queries(self) -> np.ndarray:
        c = self.cfg
        return self._memo("q", lambda: store(
            _rng(c.seed, _S_QUERY).standard_normal((c.Nq, c.W)), c.dtype))


def workload(name_or_cfg) -> Workload:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return Workload(cfg)
