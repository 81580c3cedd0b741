"""Rollout support on the CPU: the Table 7 routing policies, storage
accounting and the oracle's chunk loop, plus the library's host-only calls
(nkv_route_segments, nkv_storage_account) and the validation of the
per-layer cache calls.  No GPU needed.

Pins of the oracle (independent of its own code):
  * routing: frame counts of the deployed policies of Table 7 counted by
    hand for given history lengths;
  * storage: byte sizes of the arrays the oracle encoder really produces and
    of the codec arrays the workload generator really draws; the nominal
    coefficient ratio W*16/(r*4) of Table 5 x Table 9 (16x and 32x);
  * rollout: with an empty history the first chunk is exact attention over
    itself; later chunks equal the full or Fast read over the encodings of
    exactly the earlier chunks.
"""
import ctypes
import os

import numpy as np
import pytest

from compressed_history_attention_amd import lib, synth
from oracle import nanokv_oracle as nk
from oracle import rollout as ro

HAVE_LIB = os.path.exists(lib.LIB_PATH)
needs_lib = pytest.mark.skipif(not HAVE_LIB, reason="libnanokv.so not built")


def _full_frames(policy, n_frames):
    return [f for f in range(n_frames) if ro.frame_is_full(f, n_frames, policy)]


# ----------------------------------------------------------------------------
# routing (Table 7)
# ----------------------------------------------------------------------------

def test_hy_worldplay_policy_counts():
    # four recent frames, one anchor per 16 older frames: 64 latent frames
    # -> anchors 0, 16, 32, 48 among frames 0..59, recent 60..63
    p = ro.RoutePolicy(frame_tokens=1, recent_frames=4, anchor_every=16)
    assert _full_frames(p, 64) == [0, 16, 32, 48, 60, 61, 62, 63]
    # the listed layers anchor every eight frames: 0, 8, ..., 56 plus 60..63
    p8 = ro.RoutePolicy(frame_tokens=1, recent_frames=4, anchor_every=8)
    assert _full_frames(p8, 64) == [0, 8, 16, 24, 32, 40, 48, 56, 60, 61, 62, 63]
    # history shorter than the recent window: everything full
    assert _full_frames(p, 3) == [0, 1, 2]
    # full-layer fallback
    pf = ro.RoutePolicy(frame_tokens=1, recent_frames=4, anchor_every=16, layer_full=True)
    assert _full_frames(pf, 64) == list(range(64))


def test_lingbot_policy_counts():
    # first three chunks (3 frames each here) full; thereafter one sink frame
    # and two recent frames
    p = ro.RoutePolicy(frame_tokens=1, sink_frames=1, recent_frames=2, all_full_frames=9)
    assert _full_frames(p, 9) == list(range(9))
    assert _full_frames(p, 12) == [0, 10, 11]
    assert _full_frames(p, 24) == [0, 22, 23]
    # the full-dimensional prefix of one layer: a sink of nine frames
    pre = ro.RoutePolicy(frame_tokens=1, sink_frames=9, recent_frames=2, all_full_frames=9)
    assert _full_frames(pre, 24) == list(range(9)) + [22, 23]


def test_matrix_game_policy_counts():
    p = ro.RoutePolicy(frame_tokens=1, recent_frames=5)
    assert _full_frames(p, 20) == [15, 16, 17, 18, 19]
    assert _full_frames(p, 5) == [0, 1, 2, 3, 4]


def test_route_segments_tokens_and_ragged_frame():
    p = ro.RoutePolicy(frame_tokens=10, recent_frames=1, anchor_every=3)
    # 45 tokens = frames 0..3 of 10 tokens + ragged frame 4 of 5 tokens
    segs = ro.route_segments(p, 45)
    assert segs == [(0, 10, 0), (10, 30, 1), (30, 45, 0)]
    assert ro.route_segments(p, 0) == []
    # every token is covered exactly once and the full-token count matches
    # the frame count
    p2 = ro.RoutePolicy(frame_tokens=7, recent_frames=2, sink_frames=1, anchor_every=4)
    n = 7 * 23 + 3
    segs = ro.route_segments(p2, n)
    cov = np.zeros(n, int)
    for b, e, m in segs:
        cov[b:e] += 1
    assert (cov == 1).all()
    nf = 24
    full_tok = sum(min(n, 7 * (f + 1)) - 7 * f for f in _full_frames(p2, nf))
    assert full_tok == sum(e - b for b, e, m in segs if m == 0)
    # adjacent segments alternate modes
    assert all(segs[i][2] != segs[i + 1][2] for i in range(len(segs) - 1))


@needs_lib
def test_native_route_segments_match_oracle():
    rng = np.random.default_rng(7)
    for trial in range(300):
        p = ro.RoutePolicy(frame_tokens=int(rng.integers(1, 40)),
                           recent_frames=int(rng.integers(0, 6)),
                           sink_frames=int(rng.integers(0, 4)),
                           anchor_every=int(rng.choice([0, 1, 2, 3, 8, 16])),
                           all_full_frames=int(rng.choice([0, 0, 3, 9])),
                           layer_full=bool(rng.random() < 0.1))
        n_hist = int(rng.integers(0, 2000)) if trial else 0
        got = lib.nkv_route_segments(lib.RoutePolicy(**p.__dict__), n_hist)
        assert got == ro.route_segments(p, n_hist), (p, n_hist)


@needs_lib
def test_native_route_segments_validation():
    L = lib.load()
    n = ctypes.c_int32(-1)
    bad = lib.nkv_route_policy(0, 0, 0, 0, 0, 0)
    assert L.nkv_route_segments(ctypes.byref(bad), 10, None, 0, ctypes.byref(n)) == 1
    neg = lib.nkv_route_policy(4, -1, 0, 0, 0, 0)
    assert L.nkv_route_segments(ctypes.byref(neg), 10, None, 0, ctypes.byref(n)) == 1
    ok = lib.nkv_route_policy(4, 1, 0, 2, 0, 0)
    # too little room: EINVAL and the count needed
    buf = (lib.nkv_segment * 1)()
    assert L.nkv_route_segments(ctypes.byref(ok), 40, buf, 1, ctypes.byref(n)) == 1
    assert n.value == len(ro.route_segments(ro.RoutePolicy(4, 1, 0, 2), 40))
    assert L.nkv_route_segments(ctypes.byref(ok), -1, None, 0, ctypes.byref(n)) == 1
    assert L.nkv_route_segments(ctypes.byref(ok), 10, None, 0, None) == 1


# ----------------------------------------------------------------------------
# storage (Figure 8 split, Table 1 ratio)
# ----------------------------------------------------------------------------

def test_storage_matches_real_array_sizes():
    cfg = synth.CONFIGS["C0"]
    wl = synth.workload(cfg)
    x = wl.history_tokens(0)
    enc = nk.encode(x, wl.centers(0), wl.encoder(0), cfg.group, cfg.dtype)
    per_branch = enc["idx"].nbytes + enc["codes"].nbytes + enc["scales_bits"].nbytes
    codec = sum(a.nbytes for b in range(2) for a in (wl.centers(b), wl.encoder(b), wl.decoder(b)))
    s = ro.storage(cfg.H, cfg.d, cfg.r, cfg.group, cfg.A, cfg.A, x.shape[0], 4)
    assert s["cached"] == 2 * per_branch
    assert s["idx"] == 2 * enc["idx"].nbytes
    assert s["codes"] == 2 * enc["codes"].nbytes
    assert s["scales"] == 2 * enc["scales_bits"].nbytes
    assert s["resident"] == codec
    # uncompressed bf16 K and V of the same tokens
    assert s["original"] == 2 * x.shape[0] * cfg.W * 2


@pytest.mark.parametrize("W,r,nominal", [(16 * 128, 512, 16.0), (16 * 128, 256, 32.0),
                                         (40 * 128, 640, 32.0), (24 * 128, 384, 32.0)])
def test_nominal_ratio_table5_table9(W, r, nominal):
    H = W // 128
    s = ro.storage(H, 128, r, 32, 64, 64, 1000, 2)
    assert s["cr_nominal"] == nominal
    # stored extras (index, scales, operators) keep the effective ratio below
    assert s["cr_effective"] < s["cr_cached"] < nominal


def test_storage_long_history_limit():
    # as the history grows the resident operators amortise: the effective
    # ratio approaches original / cached = (2 W) / (4 + r/2 + 2 r/g)
    H, d, r, g = 16, 128, 256, 32
    s = ro.storage(H, d, r, g, 64, 64, 10 ** 9, 2)
    assert abs(s["cr_effective"] - 2 * H * d / (4 + r / 2 + 2 * r / g)) < 1e-3


@needs_lib
@pytest.mark.parametrize("H,d,r,g,Ak,Av,n,dt", [(16, 128, 256, 32, 64, 64, 99840, 1),
                                               (2, 16, 8, 8, 4, 4, 64, 0),
                                               (24, 128, 384, 32, 1024, 512, 0, 1),
                                               (12, 64, 192, 16, 256, 256, 12345, 0)])
def test_native_storage_matches_oracle(H, d, r, g, Ak, Av, n, dt):
    got = lib.nkv_storage_account(lib.Shape(H, d, r, g, "bf16" if dt else "f32"), Ak, Av, n)
    want = ro.storage(H, d, r, g, Ak, Av, n, 2 if dt else 4)
    for k, v in want.items():
        assert got[k] == pytest.approx(v, rel=1e-12), k


@needs_lib
def test_native_storage_validation():
    L = lib.load()
    out = lib.nkv_storage()
    sh = lib.nkv_shape(2, 16, 8, 8, 0, 0.0)
    assert L.nkv_storage_account(ctypes.byref(sh), 0, 4, 10, ctypes.byref(out)) == 1
    assert L.nkv_storage_account(ctypes.byref(sh), 4, 4, -1, ctypes.byref(out)) == 1
    assert L.nkv_storage_account(None, 4, 4, 10, ctypes.byref(out)) == 1
    assert L.nkv_storage_account(ctypes.byref(sh), 4, 4, 10, None) == 1
    bad = lib.nkv_shape(2, 16, 7, 8, 0, 0.0)
    assert L.nkv_storage_account(ctypes.byref(bad), 4, 4, 10, ctypes.byref(out)) == 1


# ----------------------------------------------------------------------------
# per-layer cache calls: validation before anything is enqueued
# ----------------------------------------------------------------------------

FAKE = 0x1000


def _cache(n_hist, capacity, A=4):
    br = lib.nkv_cache_branch(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, A)
    return lib.nkv_layer_cache(br, br, n_hist, capacity)


@needs_lib
def test_layer_append_validation():
    L = lib.load()
    sh = lib.nkv_shape(2, 16, 8, 8, 0, 0.0)
    c = _cache(10, 12)
    # no room: EINVAL, n_hist unchanged
    assert L.nkv_layer_append(ctypes.byref(sh), ctypes.byref(c), FAKE, FAKE, 3, None, 0,
                              None) == 1
    assert c.n_hist == 10
    assert L.nkv_layer_append(ctypes.byref(sh), ctypes.byref(c), FAKE, FAKE, -1, None, 0,
                              None) == 1
    # malformed descriptor
    bad = _cache(5, 4)
    assert L.nkv_layer_append(ctypes.byref(sh), ctypes.byref(bad), FAKE, FAKE, 0, None, 0,
                              None) == 1
    # NULL value rows
    assert L.nkv_layer_append(ctypes.byref(sh), ctypes.byref(c), FAKE, None, 2, None, 0,
                              None) == 1
    assert c.n_hist == 10
    # N == 0 is a no-op
    assert L.nkv_layer_append(ctypes.byref(sh), ctypes.byref(c), None, None, 0, None, 0,
                              None) == 0
    assert c.n_hist == 10
    assert L.nkv_layer_append_workspace_size(ctypes.byref(sh), ctypes.byref(bad), 1) == \
        lib.SIZE_MAX


@needs_lib
def test_layer_attend_validation():
    L = lib.load()
    sh = lib.nkv_shape(2, 16, 8, 8, 0, 0.0)
    c = _cache(40, 64)
    low = lib.nkv_route_policy(10, 1, 0, 0, 0, 0)        # frames 0..2 low
    full = lib.nkv_route_policy(10, 0, 0, 0, 0, 1)
    # part of the history low and no widths: EINVAL
    assert L.nkv_layer_attend(ctypes.byref(sh), ctypes.byref(c), ctypes.byref(low), None, FAKE,
                              4, None, None, 0, FAKE, FAKE, None, 0, None) == 1
    assert L.nkv_layer_attend_workspace_size(ctypes.byref(sh), ctypes.byref(c),
                                             ctypes.byref(low), None, 4, 0) == lib.SIZE_MAX
    # a fully routed layer needs no widths
    assert L.nkv_layer_attend_workspace_size(ctypes.byref(sh), ctypes.byref(c),
                                             ctypes.byref(full), None, 4, 0) != lib.SIZE_MAX
    bad = lib.nkv_route_policy(0, 0, 0, 0, 0, 0)
    assert L.nkv_layer_attend(ctypes.byref(sh), ctypes.byref(c), ctypes.byref(bad), None, FAKE,
                              4, None, None, 0, FAKE, FAKE, None, 0, None) == 1
    w = (ctypes.c_int32 * 2)(4, 9)                        # 9 > r
    assert L.nkv_layer_attend(ctypes.byref(sh), ctypes.byref(c), ctypes.byref(low), w, FAKE, 4,
                              None, None, 0, FAKE, FAKE, None, 0, None) == 2


# ----------------------------------------------------------------------------
# oracle rollout: reductions
# ----------------------------------------------------------------------------

def _tiny_rollout_inputs(n_layers=2, n_chunks=3, chunk=24, Nq=8):
    """Per layer a C0-style codec; per chunk and layer seeded q/k/v."""
    codecs, chunks = [], []
    wls = []
    for l in range(n_layers):
        cfg = synth.small_config("C0", seed=100 + l, n_hist=chunk * n_chunks, Nq=Nq,
                                 N_cur=chunk, chunk=chunk)
        wl = synth.workload(cfg)
        wls.append(wl)
        codecs.append(ro.LayerCodec((wl.centers(0), wl.centers(1)),
                                    (wl.encoder(0), wl.encoder(1)),
                                    (wl.decoder(0), wl.decoder(1))))
    for c in range(n_chunks):
        row = []
        for l, wl in enumerate(wls):
            rng = np.random.default_rng([5, l, c])
            q = rng.standard_normal((Nq, wl.cfg.W)).astype(np.float32)
            row.append((q, wl.history_chunk(0, c)[0], wl.history_chunk(1, c)[0]))
        chunks.append(row)
    return wls[0].cfg, codecs, chunks


def test_oracle_rollout_reductions():
    cfg, codecs, chunks = _tiny_rollout_inputs()
    pols = [ro.RoutePolicy(frame_tokens=8, layer_full=True),
            ro.RoutePolicy(frame_tokens=8, recent_frames=1, anchor_every=4)]
    outs = ro.rollout(codecs, pols, chunks, cfg.H, cfg.d, cfg.group, cfg.dtype, cfg.tau,
                      [cfg.r, [4, 6]])
    # chunk 0: no history -> exact attention over the chunk itself
    for l in range(2):
        q, k, v = (nk.as_f64(a, cfg.dtype) for a in chunks[0][l])
        o, lse = nk.exact_attention(q, k, v, cfg.H, cfg.d, cfg.tau)
        np.testing.assert_allclose(outs[0][l][0], o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(outs[0][l][1], lse, rtol=0, atol=1e-12)
    # chunk 2 of layer 0 (full layer): decode(encode(chunks 0, 1)) ; chunk 2
    l = 0
    hk = np.concatenate([chunks[c][l][1] for c in range(2)])
    hv = np.concatenate([chunks[c][l][2] for c in range(2)])
    ek = nk.encode(hk, codecs[l].centers[0], codecs[l].encoder[0], cfg.group, cfg.dtype)
    ev = nk.encode(hv, codecs[l].centers[1], codecs[l].encoder[1], cfg.group, cfg.dtype)
    kdec = nk.decode(ek["idx"], ek["codes"], ek["scales_bits"],
                     nk.as_f64(codecs[l].centers[0], cfg.dtype),
                     nk.as_f64(codecs[l].decoder[0], cfg.dtype), cfg.group)
    vdec = nk.decode(ev["idx"], ev["codes"], ev["scales_bits"],
                     nk.as_f64(codecs[l].centers[1], cfg.dtype),
                     nk.as_f64(codecs[l].decoder[1], cfg.dtype), cfg.group)
    q, k, v = (nk.as_f64(a, cfg.dtype) for a in chunks[2][l])
    o, lse = nk.exact_attention(q, np.concatenate([kdec, k]), np.concatenate([vdec, v]),
                                cfg.H, cfg.d, cfg.tau)
    np.testing.assert_allclose(outs[2][l][0], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[2][l][1], lse, rtol=0, atol=1e-12)
    # the Fast layer at chunk 2: 48 history tokens = 6 frames of 8; frames 0
    # and 4 anchors, frame 5 recent -> low frames 1-3
    l = 1
    hk = np.concatenate([chunks[c][l][1] for c in range(2)])
    hv = np.concatenate([chunks[c][l][2] for c in range(2)])
    ek = nk.encode(hk, codecs[l].centers[0], codecs[l].encoder[0], cfg.group, cfg.dtype)
    ev = nk.encode(hv, codecs[l].centers[1], codecs[l].encoder[1], cfg.group, cfg.dtype)
    kb = nk.Branch(ek["idx"], ek["codes"], ek["scales_bits"], codecs[l].centers[0],
                   codecs[l].decoder[0], cfg.dtype, cfg.group)
    vb = nk.Branch(ev["idx"], ev["codes"], ev["scales_bits"], codecs[l].centers[1],
                   codecs[l].decoder[1], cfg.dtype, cfg.group)
    q, k, v = (nk.as_f64(a, cfg.dtype) for a in chunks[2][l])
    segs = [(0, 8, 0), (8, 32, 1), (32, 48, 0)]
    assert ro.route_segments(pols[1], 48) == segs
    o, lse = nk.attend_fast(q, kb, vb, segs, [4, 6], k, v, cfg.H, cfg.d, cfg.tau)
    np.testing.assert_allclose(outs[2][l][0], o, rtol=0, atol=1e-12)
    # and it differs from the full read (the low part is really low-dimensional)
    of, _ = nk.attend_full(q, kb, vb, k, v, cfg.H, cfg.d, cfg.tau)
    assert np.abs(of - o).max() > 1e-3
