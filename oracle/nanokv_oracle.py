"""fp64 CPU oracle for compressed-history attention (NanoKV).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library: it reads the stored bits of its inputs itself and computes
everything in float64 with numpy (matmul as the only library primitive, plus
``scipy.sparse`` for one-hot sums).

What it computes follows the NanoKV pages
(NanoKV: High-Ratio KV Cache Compression for Autoregressive Video Generation):

* abstract: historical K/V are stored as shared cluster centers plus joint
  head-channel residual coefficients in low-bit form; the Fast variant reuses
  the stored coefficients for mixed-dimensional attention;
* Figure 4(a): K/V history is stored as coefficients and shared centers and is
  read either full-dimensionally or mixed-dimensionally;
* Figure 4(b): the encoder compresses residuals into INT4 coefficients, the
  decoder reconstructs them and adds the centers back;
* Figure 4(d): a fixed policy routes history to full- or low-dimensional
  attention; the low-dimensional part reduces the queries and restores the
  output dimension before LSE merging;
* Table 5 caption: rank is per layer and per K/V branch, centers are fitted
  separately for K and V.

Readings taken where the pages are silent (each is listed in the design
notes): squared-L2 nearest center with ties to the lowest index; INT4 groups
are ``g`` consecutive coefficients of one token with an fp16 scale equal to
max|z|/7 rounded half-to-even, codes rounded half-to-even and clamped to
[-8, 7], two's-complement nibbles with coefficient 2j in the low nibble of
byte j; the softmax scale multiplies the whole score (center term included);
LSE uses the natural log; no masking; the low-dimensional read truncates both
K and V coefficients to their leading ``r_low`` entries.

Parity status: every function here is pinned by tests under ``tests/``
(closed forms, textbook special cases, brute force on tiny inputs); nothing
is "parity unpinned" except agreement with the pages' *fitted* codec
(trained encoders, decoders, centers), which the pages do not print.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np
import scipy.sparse as sp

F32, BF16 = "f32", "bf16"


# ----------------------------------------------------------------------------
# reading stored tensors (oracle-local; bit-exact upcasts)
# ----------------------------------------------------------------------------

def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> float64.  bf16 tensors are uint16 bit patterns."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------------------
# encoder: Figure 4(b) -- nearest center, residual, linear encoder, INT4
# ----------------------------------------------------------------------------

def assign(x: np.ndarray, centers: np.ndarray, block: int = 2048) -> np.ndarray:
    """Index of the nearest center (squared L2) per token; ties -> lowest index.

    x [N, W] and centers [A, W] are float64.  Uses ||mu||^2 - 2 x.mu (the
    per-token ||x||^2 does not change the argmin); see ``assign_direct`` for
    the direct-difference form used on tiny inputs.
    """
    n = x.shape[0]
    out = np.empty(n, dtype=np.int32)
    mu2 = np.einsum("aw,aw->a", centers, centers)
    for s in range(0, n, block):
        dist = mu2[None, :] - 2.0 * (x[s:s + block] @ centers.T)
        out[s:s + block] = np.argmin(dist, axis=1)  # first minimum = lowest index
    return out


def assign_direct(x: np.ndarray, centers: np.ndarray) -> np.ndarray:
    """Direct sum of squared differences (small inputs)."""
    diff = x[:, None, :] - centers[None, :, :]
    return np.argmin(np.sum(diff * diff, axis=2), axis=1).astype(np.int32)


def project(x: np.ndarray, centers: np.ndarray, idx: np.ndarray,
            encoder: np.ndarray) -> np.ndarray:
    """Residual coefficients z = E (x - mu[idx]); E is [r, W]."""
    return (x - centers[idx]) @ encoder.T


def _fp16_neighbours(u: np.ndarray):
    s = u.astype(np.float16)
    s64 = s.astype(np.float64)
    up = np.nextafter(s, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(s, np.float16(-np.inf)).astype(np.float64)
    other = np.where(s64 >= u, dn, up)
    return s64, other


def quantize(z: np.ndarray, group: int):
    """INT4 quantisation of coefficient groups (Figure 4(b), "INT4 coefficients").

    z [N, r] float64, ``group`` consecutive coefficients of one token share a
    scale s = fp16_rne(max|z| / 7).  code = clamp(rint(z / s), -8, 7) with
    rint half-to-even; s == 0 gives all-zero codes.  Returns
    (codes int8 [N, r], scales float16 [N, r/group], boundary mask [N, r],
    scale-near mask [N, r/group]).  The boundary mask marks codes whose
    pre-round value lies within 1e-3 of a .5 boundary; the scale-near mask
    marks groups whose max|z|/7 lies within 1e-5 (relative) of an fp16
    rounding midpoint.
    """
    n, r = z.shape
    if r % group:
        raise ValueError("r must be a multiple of the group size")
    zg = z.reshape(n, r // group, group)
    m = np.max(np.abs(zg), axis=2)
    u = m / 7.0
    with np.errstate(over="ignore"):
        s16 = u.astype(np.float16)          # fp64 -> fp16, round half to even
    s = s16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s[..., None] > 0, zg / s[..., None], 0.0)
    codes = np.clip(np.rint(v), -8, 7).astype(np.int8)
    frac = v - np.floor(v)
    boundary = np.abs(frac - 0.5) < 1e-3
    with np.errstate(over="ignore", invalid="ignore"):
        s_near, s_other = _fp16_neighbours(u)
        mid = 0.5 * (s_near + s_other)
        scale_near = np.isfinite(mid) & (np.abs(u - mid) <= 1e-5 * u) & (u > 0)
    return (codes.reshape(n, r), s16, boundary.reshape(n, r), scale_near)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles; coefficient 2j -> low nibble of byte j."""
    c = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray, r: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    out = np.empty((p.shape[0], r), dtype=np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def encode(x_stored: np.ndarray, centers_stored: np.ndarray,
           encoder_stored: np.ndarray, group: int, dtype: str,
           block: int = 4096) -> dict:
    """Full encoder: nearest center -> residual -> E projection -> INT4.

    Returns idx int32 [N], codes uint8 [N, r/2], scales uint16 (fp16 bits)
    [N, r/group], plus ``codes_int`` int8 [N, r], ``z`` float64 [N, r] and the
    boundary / scale-near masks used by the parity rules.
    """
    mu = as_f64(centers_stored, dtype)
    enc = as_f64(encoder_stored, dtype)
    n = x_stored.shape[0]
    r = enc.shape[0]
    out = {k: [] for k in ("idx", "z", "codes_int", "scales", "boundary", "scale_near")}
    for s in range(0, n, block):
        x = as_f64(x_stored[s:s + block], dtype)
        idx = assign(x, mu)
        z = project(x, mu, idx, enc)
        codes, s16, bnd, snear = quantize(z, group)
        for k, v in (("idx", idx), ("z", z), ("codes_int", codes), ("scales", s16),
                     ("boundary", bnd), ("scale_near", snear)):
            out[k].append(v)
    if n == 0:
        res = dict(idx=np.zeros(0, np.int32), z=np.zeros((0, r)),
                   codes_int=np.zeros((0, r), np.int8),
                   scales=np.zeros((0, r // group), np.float16),
                   boundary=np.zeros((0, r), bool),
                   scale_near=np.zeros((0, r // group), bool))
    else:
        res = {k: np.concatenate(v, axis=0) for k, v in out.items()}
    res["codes"] = pack_int4(res["codes_int"])
    res["scales_bits"] = res["scales"].view(np.uint16)
    return res


# ----------------------------------------------------------------------------
# decoder: Figure 4(b) -- dequantise, linear decoder, add the center back
# ----------------------------------------------------------------------------

def dequantize(codes_packed: np.ndarray, scales_bits: np.ndarray, r: int,
               group: int) -> np.ndarray:
    """c_hat = code * scale, float64 [N, r]."""
    c = unpack_int4(codes_packed, r).astype(np.float64)
    s = fp16_bits_to_f64(scales_bits)
    return c * np.repeat(s, group, axis=1)


def decode(idx: np.ndarray, codes_packed: np.ndarray, scales_bits: np.ndarray,
           centers: np.ndarray, decoder: np.ndarray, group: int) -> np.ndarray:
    """x_hat = mu[idx] + D c_hat.  centers [A, W], decoder [W, r] float64."""
    r = decoder.shape[1]
    ch = dequantize(codes_packed, scales_bits, r, group)
    return centers[idx] + ch @ decoder.T


# ----------------------------------------------------------------------------
# attention and LSE merging
# ----------------------------------------------------------------------------

def exact_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, H: int,
                    d: int, tau: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention per head, no mask.

    q [Nq, H*d], k/v [Nk, H*d] float64.  Channel h*d + j belongs to head h.
    Returns O [Nq, H*d] and LSE [Nq, H] (natural log).  An empty key set
    gives O = 0 and LSE = -inf.
    """
    nq = q.shape[0]
    o = np.zeros((nq, H * d))
    lse = np.full((nq, H), -np.inf)
    if k.shape[0] == 0 or nq == 0:
        return o, lse
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        s = tau * (q[:, sl] @ k[:, sl].T)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        o[:, sl] = (p @ v[:, sl]) / l
        lse[:, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def lse_merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]], H: int, d: int):
    """Merge partial attentions (O_i, LSE_i) over disjoint key sets.

    L = log(sum_i exp(L_i)),  O = sum_i exp(L_i - L) O_i.  Parts with
    LSE = -inf contribute nothing; if every part is -inf the result is
    O = 0, L = -inf.
    """
    nq = parts[0][0].shape[0]
    lses = np.stack([p[1] for p in parts], axis=0)          # [P, Nq, H]
    mx = np.max(lses, axis=0)
    fin = np.isfinite(mx)
    ref = np.where(fin, mx, 0.0)
    with np.errstate(invalid="ignore"):
        tot = np.sum(np.exp(lses - ref[None]), axis=0)     # exp(-inf) = 0
    L = np.full(mx.shape, -np.inf)
    L[fin] = ref[fin] + np.log(tot[fin])
    o = np.zeros((nq, H * d))
    for oi, li in parts:
        w = np.zeros(li.shape)
        ok = fin & np.isfinite(li)
        w[ok] = np.exp(li[ok] - L[ok])
        o += np.repeat(w, d, axis=1) * oi
    return o, L


# ----------------------------------------------------------------------------
# compressed history (one K or V branch) and the two readers
# ----------------------------------------------------------------------------

class Branch:
    """Compressed history of one branch as stored: idx, packed codes, scales,
    plus the branch's centers [A, W] and decoder [W, r] (float64 copies)."""

    def __init__(self, idx, codes, scales_bits, centers_stored, decoder_stored,
                 dtype: str, group: int):
        self.idx = np.asarray(idx, dtype=np.int32)
        self.codes = np.asarray(codes, dtype=np.uint8)
        self.scales = np.asarray(scales_bits, dtype=np.uint16)
        self.centers = as_f64(centers_stored, dtype)
        self.decoder = as_f64(decoder_stored, dtype)
        self.group = group

    @property
    def r(self) -> int:
        return self.decoder.shape[1]

    def rows(self, sel) -> "Branch":
        b = object.__new__(Branch)
        b.idx, b.codes, b.scales = self.idx[sel], self.codes[sel], self.scales[sel]
        b.centers, b.decoder, b.group = self.centers, self.decoder, self.group
        return b

    def decode(self) -> np.ndarray:
        return decode(self.idx, self.codes, self.scales, self.centers,
                      self.decoder, self.group)

    def coefficients(self) -> np.ndarray:
        return dequantize(self.codes, self.scales, self.r, self.group)


def attend_full(q: np.ndarray, kb: Branch, vb: Branch, cur_k: np.ndarray,
                cur_v: np.ndarray, H: int, d: int, tau: float):
    """NanoKV full-dimensional read (Figure 4(a)): decode every history token,
    then ordinary softmax attention over [decoded history ; current chunk]."""
    k = np.concatenate([kb.decode(), cur_k], axis=0)
    v = np.concatenate([vb.decode(), cur_v], axis=0)
    return exact_attention(q, k, v, H, d, tau)


def head_widths(r_low, H: int) -> list:
    """Per-head low-dimensional width: one int for every head, or one per head
    (the deployed configurations of Table 6 mix 32, 64, 96 and 128)."""
    if np.ndim(r_low) == 0:
        return [int(r_low)] * H
    widths = [int(x) for x in r_low]
    if len(widths) != H:
        raise ValueError("need one r_low per head")
    return widths


def low_attention(q: np.ndarray, kb: Branch, vb: Branch, r_low, H: int,
                  d: int, tau: float, qblock: int = 256, maps=None):
    """Low-dimensional read of a history partition (Figure 4(d)).

    Per head h, with D_{X,h} the rows h*d..h*d+d-1 of decoder X and [:r_low]
    the leading coefficients (r_low may differ per head, Table 6):
      q~     = D_{K,h}[:, :r_low]^T q_h                  (query reduction)
      s_t    = tau * (q~ . c^K_t[:r_low] + q_h . mu^K_{a^K_t, h})
      p      = softmax_t(s)
      O_h    = D_{V,h}[:, :r_low] sum_t p_t c^V_t[:r_low]
               + sum_t p_t mu^V_{a^V_t, h}                 (output restoration)
      LSE_h  = logsumexp_t(s)
    With r_low = r this equals decoding followed by exact attention.

    ``maps`` = (Q, O), float64 [W, ld] each, replaces D_K in the query
    reduction and D_V in the restoration by other maps (Table 8 compares the
    analytical decoder maps with adapted ones); the scores still use the
    stored K coefficients and centers.
    """
    nq = q.shape[0]
    nl = kb.idx.shape[0]
    o = np.zeros((nq, H * d))
    lse = np.full((nq, H), -np.inf)
    if nl == 0 or nq == 0:
        return o, lse
    widths = head_widths(r_low, H)
    ck_all = kb.coefficients()
    cv_all = vb.coefficients()
    A_v = vb.centers.shape[0]
    onehot_v = sp.csr_matrix((np.ones(nl), (np.arange(nl), vb.idx)), shape=(nl, A_v))
    for h in range(H):
        rl = widths[h]
        ck = ck_all[:, :rl]
        cv = cv_all[:, :rl]
        sl = slice(h * d, (h + 1) * d)
        dk = (kb.decoder if maps is None else maps[0])[sl, :rl]
        dv = (vb.decoder if maps is None else maps[1])[sl, :rl]
        muk = kb.centers[:, sl]
        muv = vb.centers[:, sl]
        for s0 in range(0, nq, qblock):
            qh = q[s0:s0 + qblock, sl]
            qt = qh @ dk                                  # [b, r_low]
            tk = qh @ muk.T                               # [b, A_k] center scores
            s = tau * (qt @ ck.T + tk[:, kb.idx])
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            acc = p @ cv                                  # coefficient-space sum
            wmass = np.asarray((sp.csr_matrix(p) @ onehot_v).todense())  # [b, A_v]
            o[s0:s0 + qblock, sl] = (acc @ dv.T + wmass @ muv) / l
            lse[s0:s0 + qblock, h] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def route_indices(segments: Sequence[Tuple[int, int, int]], n_hist: int):
    """Split history positions into (full-routed, low-routed) index arrays.
    segments: (begin, end, mode) with mode 0 = full, 1 = low; they must be
    disjoint and cover [0, n_hist)."""
    full, low = [], []
    covered = np.zeros(n_hist, dtype=np.int32)
    for b, e, m in segments:
        if not (0 <= b <= e <= n_hist):
            raise ValueError("segment out of range")
        covered[b:e] += 1
        (full if m == 0 else low).append(np.arange(b, e))
    if n_hist and not np.all(covered == 1):
        raise ValueError("segments must be disjoint and cover the history")
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, dtype=np.int64)
    return cat(full), cat(low)


def attend_fast(q: np.ndarray, kb: Branch, vb: Branch, segments, r_low,
                cur_k: np.ndarray, cur_v: np.ndarray, H: int, d: int,
                tau: float, maps=None):
    """NanoKV-Fast (Figure 4(d)): full-routed history plus the current chunk
    through decode + exact attention, low-routed history through
    ``low_attention`` (one width for all heads, or one per head as in the
    deployed configurations of Table 6; optional query-reduction and
    restoration maps, Table 8), then LSE merging of the two parts."""
    n_hist = kb.idx.shape[0]
    full, low = route_indices(segments, n_hist)
    kf = np.concatenate([kb.rows(full).decode(), cur_k], axis=0)
    vf = np.concatenate([vb.rows(full).decode(), cur_v], axis=0)
    part_full = exact_attention(q, kf, vf, H, d, tau)
    part_low = low_attention(q, kb.rows(low), vb.rows(low), r_low, H, d, tau, maps=maps)
    return lse_merge([part_full, part_low], H, d)
