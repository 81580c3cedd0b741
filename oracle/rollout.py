"""fp64 CPU oracle for the multi-layer rollout: routing policy, storage
accounting and the chunk loop (test infrastructure only).

TEST INFRASTRUCTURE ONLY, like ``nanokv_oracle``: nothing in the product path
imports or calls it; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may.  It shares no code with the HIP
library.

What it follows on the NanoKV pages
(NanoKV: High-Ratio KV Cache Compression for Autoregressive Video Generation):

* Table 7 (full-dimensional routing of the deployed Fast configurations): a
  fixed, per-layer policy sends some history frames to the full-dimensional
  read -- a window of recent latent frames, periodic anchors among older
  frames, sink frames at the start of the history, all of the history while
  it is still short ("first three chunks"), or the whole layer ("full-layer
  fallback");
* Figure 8 / Table 1: persistent KV storage split into cached data and
  resident operators, and the effective KV compression ratio (original KV
  bytes over compressed bytes);
* Figure 4(a)/(b): every finished chunk is encoded and appended to the
  history, which every later chunk reads.

Readings taken where the pages are silent (each is listed in the design
notes):

* history positions are grouped into latent frames of ``frame_tokens``
  consecutive tokens, oldest first; a ragged last frame is a frame;
* "one anchor per F older frames": among frames older than the recent window
  and not sinks, frame ``f`` is an anchor when ``f % F == 0`` (frame indices
  count from the start of the history, so a frame's route never changes once
  it has left the recent window);
* "first N chunks" full: while the history holds at most ``all_full_frames``
  frames, every frame is read full;
* storage counts what the stored format holds: per token and branch a 4-byte
  center index, r/2 bytes of packed codes and r/group fp16 scales (cached
  data); per layer and branch the centers [A, W], encoder [r, W] and decoder
  [W, r] at the element size of the codec dtype (resident operators); the
  uncompressed reference is K and V in bf16 (2 bytes per value).

Parity status: ``frame_is_full`` is pinned by hand-counted cases of the
Table 7 policies; ``storage`` by the byte sizes of arrays the oracle encoder
actually produces and by the nominal-ratio closed form; ``rollout`` by the
single-chunk reduction to ``attend_fast``/``attend_full`` and by brute force.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from . import nanokv_oracle as nk


@dataclass(frozen=True)
class RoutePolicy:
    """Per-layer full-dimensional routing (Table 7)."""
    frame_tokens: int          # tokens per latent frame (> 0)
    recent_frames: int = 0     # most recent frames read full
    sink_frames: int = 0       # first frames of the history read full
    anchor_every: int = 0      # one anchor per this many older frames (0: none)
    all_full_frames: int = 0   # history of at most this many frames: all full
    layer_full: bool = False   # full-layer fallback


def frame_is_full(f: int, n_frames: int, p: RoutePolicy) -> bool:
    """Route of latent frame ``f`` of a history of ``n_frames`` frames."""
    if p.layer_full or n_frames <= p.all_full_frames:
        return True
    if f < p.sink_frames:
        return True
    if f >= n_frames - p.recent_frames:
        return True
    return p.anchor_every > 0 and f % p.anchor_every == 0


def route_segments(p: RoutePolicy, n_hist: int) -> List[Tuple[int, int, int]]:
    """Token-level (begin, end, mode) ranges, mode 0 = full and 1 = low,
    adjacent ranges of one mode joined."""
    if p.frame_tokens <= 0:
        raise ValueError("frame_tokens must be positive")
    n_frames = -(-n_hist // p.frame_tokens)
    segs: List[Tuple[int, int, int]] = []
    for f in range(n_frames):
        b = f * p.frame_tokens
        e = min(n_hist, b + p.frame_tokens)
        m = 0 if frame_is_full(f, n_frames, p) else 1
        if segs and segs[-1][2] == m and segs[-1][1] == b:
            segs[-1] = (segs[-1][0], e, m)
        else:
            segs.append((b, e, m))
    return segs


def storage(H: int, d: int, r: int, group: int, A_k: int, A_v: int,
            n_hist: int, codec_elem_bytes: int) -> dict:
    """Bytes one layer keeps for ``n_hist`` history tokens (Figure 8 split)."""
    W = H * d
    per_token = 4 + r // 2 + 2 * (r // group)       # idx + codes + scales
    cached = 2 * n_hist * per_token                 # K and V branches
    centers = (A_k + A_v) * W * codec_elem_bytes
    encoders = 2 * r * W * codec_elem_bytes
    decoders = 2 * W * r * codec_elem_bytes
    resident = centers + encoders + decoders
    original = 2 * n_hist * W * 2                   # bf16 K and V
    return {
        "idx": 2 * n_hist * 4,
        "codes": 2 * n_hist * (r // 2),
        "scales": 2 * n_hist * 2 * (r // group),
        "cached": cached,
        "centers": centers,
        "encoders": encoders,
        "decoders": decoders,
        "resident": resident,
        "total": cached + resident,
        "original": original,
        "cr_effective": original / (cached + resident) if cached + resident else 0.0,
        "cr_cached": original / cached if cached else 0.0,
        "cr_nominal": (W * 16) / (r * 4),
    }


@dataclass
class LayerCodec:
    """Stored codec of one layer: per branch centers, encoder, decoder."""
    centers: Tuple[np.ndarray, np.ndarray]
    encoder: Tuple[np.ndarray, np.ndarray]
    decoder: Tuple[np.ndarray, np.ndarray]


def rollout(codecs: Sequence[LayerCodec], policies: Sequence[RoutePolicy],
            chunks, H: int, d: int, group: int, dtype: str, tau: float,
            r_low) -> list:
    """Chunk loop of an autoregressive rollout without a backbone.

    ``chunks[c][l]`` holds the (queries, keys, values) of chunk ``c`` at layer
    ``l`` in storage dtype.  For every chunk and layer the queries attend to
    [history ; the chunk's own keys/values] -- Fast routing by the layer's
    policy, or the full read when the policy sends everything full -- and the
    finished chunk's K and V are then encoded and appended to that layer's
    history.  Returns ``out[c][l] = (O, LSE)``.  ``r_low`` is one width or
    one list of per-head widths per layer.
    """
    L = len(codecs)
    hist = [[[], []] for _ in range(L)]       # per layer, per branch: encodings
    outs = []
    for chunk in chunks:
        row = []
        for l in range(L):
            q, kc, vc = chunk[l]
            cod = codecs[l]
            br = []
            for b in range(2):
                parts = hist[l][b]
                r = cod.decoder[b].shape[1]
                if parts:
                    idx = np.concatenate([p[0] for p in parts])
                    codes = np.concatenate([p[1] for p in parts])
                    scales = np.concatenate([p[2] for p in parts])
                else:
                    idx = np.zeros(0, np.int32)
                    codes = np.zeros((0, r // 2), np.uint8)
                    scales = np.zeros((0, r // group), np.uint16)
                br.append(nk.Branch(idx, codes, scales, cod.centers[b],
                                    cod.decoder[b], dtype, group))
            n_hist = br[0].idx.shape[0]
            qf = nk.as_f64(q, dtype)
            kf = nk.as_f64(kc, dtype)
            vf = nk.as_f64(vc, dtype)
            segs = route_segments(policies[l], n_hist)
            if all(m == 0 for _, _, m in segs):
                res = nk.attend_full(qf, br[0], br[1], kf, vf, H, d, tau)
            else:
                rl = r_low[l] if isinstance(r_low, (list, tuple)) else r_low
                res = nk.attend_fast(qf, br[0], br[1], segs, rl, kf, vf, H, d, tau)
            row.append(res)
            for b, x in ((0, kc), (1, vc)):
                enc = nk.encode(x, cod.centers[b], cod.encoder[b], group, dtype)
                hist[l][b].append((enc["idx"], enc["codes"], enc["scales_bits"]))
        outs.append(row)
    return outs
