"""Shared set-up of the GPU parity tests: seeded workloads, their
oracle-encoded histories, device uploads and the parity rules."""
from __future__ import annotations

import functools
import sys
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
from compressed_history_attention_amd import lib, synth


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))


def to_dev(a: np.ndarray, dtype: Optional[str] = None) -> torch.Tensor:
    if dtype is not None:
        t = to_torch(a, dtype)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def shape_of(cfg: synth.Config) -> lib.Shape:
    return lib.Shape(cfg.H, cfg.d, cfg.r, cfg.group, cfg.dtype)


@dataclass
class Case:
    cfg: synth.Config
    w: synth.Workload
    enc: List[dict]                # per branch: oracle encoding of the full attended history
    new_enc: Optional[List[dict]]  # per branch: oracle encoding of the appended chunk


def _encode_history(w: synth.Workload, b: int) -> dict:
    cfg = w.cfg
    parts = []
    for k in range(w.n_history_chunks()):
        x = w.history_chunk(b, k)[0]
        parts.append(oracle.encode(x, w.centers(b), w.encoder(b), cfg.group, cfg.dtype))
    keys = ("idx", "codes", "scales_bits")
    if not parts:
        return {"idx": np.zeros(0, np.int32), "codes": np.zeros((0, cfg.r // 2), np.uint8),
                "scales_bits": np.zeros((0, cfg.r // cfg.group), np.uint16)}
    return {k: np.concatenate([p[k] for p in parts]) for k in keys}


@functools.lru_cache(maxsize=None)
def get_case(cfg: synth.Config) -> Case:
    w = synth.workload(cfg)
    enc = [_encode_history(w, b) for b in range(2)]
    new_enc = None
    if cfg.n_new:
        new_enc = []
        for b in range(2):
            x = w.new_chunk(b)[0]
            new_enc.append(oracle.encode(x, w.centers(b), w.encoder(b), cfg.group, cfg.dtype))
    return Case(cfg, w, enc, new_enc)


def oracle_branch(case: Case, b: int, include_new: bool = True) -> oracle.Branch:
    cfg = case.cfg
    e = case.enc[b]
    idx, codes, sc = e["idx"], e["codes"], e["scales_bits"]
    if include_new and case.new_enc is not None:
        n = case.new_enc[b]
        idx = np.concatenate([idx, n["idx"]])
        codes = np.concatenate([codes, n["codes"]])
        sc = np.concatenate([sc, n["scales_bits"]])
    return oracle.Branch(idx, codes, sc, case.w.centers(b), case.w.decoder(b), cfg.dtype, cfg.group)


def device_branch(case: Case, b: int, include_new: bool = True) -> lib.Branch:
    ob = oracle_branch(case, b, include_new)
    cfg = case.cfg
    return lib.Branch(to_dev(ob.idx), to_dev(ob.codes), to_dev(ob.scales),
                      to_dev(case.w.centers(b), cfg.dtype), to_dev(case.w.decoder(b), cfg.dtype))


QBLOCK = 128  # the smallest query block of any kernel (flash's 4-wave blocks)


def q_rows(cfg: synth.Config, n_sample: Optional[int], seed: int = 0) -> np.ndarray:
    """Query rows compared against the oracle: all of them (n_sample None),
    or a stratified sample that reaches every 128-row query block -- its
    first row, its last row and max(1, n_sample // blocks) seeded random rows
    inside it -- so every block of every kernel (128- and 256-row blocks, the
    ragged last block) has rows under test."""
    if n_sample is None or n_sample >= cfg.Nq:
        return np.arange(cfg.Nq)
    rng = np.random.default_rng(seed)
    nb = (cfg.Nq + QBLOCK - 1) // QBLOCK
    per = max(1, n_sample // nb)
    rows = set()
    for b in range(nb):
        lo, hi = b * QBLOCK, min(cfg.Nq, (b + 1) * QBLOCK)
        rows |= {lo, hi - 1}
        rows |= set(rng.integers(lo, hi, size=per).tolist())
    return np.array(sorted(rows))


def oracle_inputs(case: Case, rows: np.ndarray):
    cfg = case.cfg
    q = oracle.as_f64(case.w.queries()[rows], cfg.dtype)
    ck = oracle.as_f64(case.w.current(0), cfg.dtype) if cfg.N_cur else np.zeros((0, cfg.W))
    cv = oracle.as_f64(case.w.current(1), cfg.dtype) if cfg.N_cur else np.zeros((0, cfg.W))
    return q, ck, cv


def oracle_full_chunked(q, kb: oracle.Branch, vb: oracle.Branch, ck, cv, cfg, chunk=8192):
    """Full-dimensional read computed chunk by chunk and LSE-merged (equal to
    oracle.attend_full by the merge = concatenation pin), bounded memory."""
    n = kb.idx.shape[0]
    parts = []
    for s in range(0, n, chunk):
        sel = np.arange(s, min(n, s + chunk))
        parts.append(oracle.exact_attention(q, kb.rows(sel).decode(), vb.rows(sel).decode(),
                                            cfg.H, cfg.d, cfg.tau))
    parts.append(oracle.exact_attention(q, ck, cv, cfg.H, cfg.d, cfg.tau))
    return oracle.lse_merge(parts, cfg.H, cfg.d)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def attention_errors(out: np.ndarray, lse: np.ndarray, ref_o: np.ndarray, ref_l: np.ndarray):
    rel = float(np.max(np.abs(out - ref_o)) / max(np.max(np.abs(ref_o)), 1e-30))
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(lse)), "LSE finiteness differs"
    lerr = float(np.max(np.abs(lse[fin] - ref_l[fin]))) if fin.any() else 0.0
    return rel, lerr


def check_encode(gidx, gcodes, gscales, ref: dict, group: int):
    """Parity rules of the encoder.

    * indices bit-exact;
    * scales bit-exact except groups flagged scale-near, where the GPU scale
      must be one of the two fp16 neighbours and the GPU codes must equal the
      oracle codes recomputed with the GPU scale;
    * codes bit-exact except where the oracle's pre-round value lies within
      1e-3 of a rounding boundary (there |difference| <= 1).
    Returns counts for the report.
    """
    assert np.array_equal(gidx, ref["idx"]), \
        f"center indices differ at {np.flatnonzero(gidx != ref['idx'])[:10]}"
    n, ng = ref["scales"].shape
    r = ng * group
    gs = gscales.view(np.uint16)
    rs = ref["scales_bits"]
    near = ref["scale_near"]
    bad_scale = (gs != rs) & ~near
    assert not bad_scale.any(), f"{bad_scale.sum()} scales differ outside the near-midpoint window"
    gc = oracle.unpack_int4(gcodes, r).astype(np.int64)
    rc = ref["codes_int"].astype(np.int64).copy()
    flipped = np.argwhere(gs != rs)
    z = ref["z"]
    for t, g in flipped:
        s_gpu = float(gs[t, g:g + 1].view(np.float16)[0])
        s_or = float(rs[t, g:g + 1].view(np.float16)[0])
        lo, hi = sorted((s_or, float(np.nextafter(np.float16(s_or), np.float16(np.inf)))))
        dn = float(np.nextafter(np.float16(s_or), np.float16(-np.inf)))
        assert s_gpu in (lo, hi, dn), "scale is not an fp16 neighbour of the oracle's"
        v = z[t, g * group:(g + 1) * group] / s_gpu
        rc[t, g * group:(g + 1) * group] = np.clip(np.rint(v), -8, 7)
    diff = gc != rc
    allowed = ref["boundary"]
    assert not (diff & ~allowed).any(), \
        f"{(diff & ~allowed).sum()} codes differ outside the rounding window"
    assert np.all(np.abs(gc - rc)[diff] <= 1)
    return {"scale_flips": int(len(flipped)), "near_groups": int(near.sum()),
            "code_diffs": int(diff.sum()), "window_codes": int(allowed.sum()),
            "codes": int(rc.size)}
