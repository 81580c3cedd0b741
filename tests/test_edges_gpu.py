"""GPU tests of paths the workload generator never reaches by itself, through
the C ABI, against the fp64 oracle:

* a Fast call whose route sends nothing low-dimensional, with widths the
  tuned low-dimensional kernels do not serve (the workspace it uses must be
  the one its size query returns: guard bytes after it stay untouched);
* the LSE merge with a head dimension that is not a multiple of four and
  with the output written over an input (fp32);
* nearest-center assignment with exact duplicates (lowest index wins) and
  near-ties a single bf16 step apart, where fp32 distances cannot decide and
  the exact fallback must give the exact-arithmetic argmin;
* low-dimensional rows whose score bound would be too loose (large queries):
  the kernels recompute those rows exactly;
* the generic kernels (nkv_force_generic) on the full C2 workload.
"""
import dataclasses
import fractions

import numpy as np
import pytest
import torch

import oracle
from compressed_history_attention_amd import lib, synth
from gpu_cases import (attention_errors, check_encode, device_branch, from_dev, get_case, log,
                       oracle_branch, oracle_full_chunked, oracle_inputs, q_rows, shape_of,
                       to_dev)

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 1e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# all-full routes with widths the tuned low-dimensional kernels do not serve
# --------------------------------------------------------------------------

BASE = synth.small_config("C2", H=2, A=200, n_hist=2000, Nq=100, N_cur=50, chunk=700, r_low=48,
                          n_full_tail=700)


@pytest.mark.parametrize("r_low", [24, 192])
def test_fast_all_full_route_unserved_width(r_low):
    cfg = BASE
    case = get_case(cfg)
    shape = shape_of(cfg)
    kb, vb = device_branch(case, 0), device_branch(case, 1)
    q = to_dev(case.w.queries(), cfg.dtype)
    ck, cv = to_dev(case.w.current(0), cfg.dtype), to_dev(case.w.current(1), cfg.dtype)
    route = [(0, cfg.n_attend, 0)]
    need = lib.nkv_attend_workspace_size(shape, cfg.A, cfg.A, cfg.n_attend, route, r_low, cfg.Nq,
                                         cfg.N_cur)
    guard = 1 << 16
    buf = torch.full((need + guard,), 0xAB, dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.Nq, cfg.W), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((cfg.Nq, cfg.H), dtype=torch.float32, device="cuda")
    log(f"all-full route r_low={r_low}: workspace {need} B + {guard} guard bytes")
    lib.nkv_attend_fast(shape, kb, vb, cfg.n_attend, route, r_low, q, ck, cv, out, lse,
                        ws=buf[:need])
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xAB).all()), "the call wrote past its workspace"
    rows = np.arange(cfg.Nq)
    qo, cko, cvo = oracle_inputs(case, rows)
    ro, rl = oracle_full_chunked(qo, oracle_branch(case, 0), oracle_branch(case, 1), cko, cvo, cfg)
    rel, lerr = attention_errors(from_dev(out), from_dev(lse), ro, rl)
    log(f"  rel={rel:.3e} dLSE={lerr:.3e}")
    assert rel <= OUT_TOL and lerr <= LSE_TOL


# --------------------------------------------------------------------------
# LSE merge: scalar path and in-place fp32 output
# --------------------------------------------------------------------------

def _merge_inputs(Nq, H, d, seed=3):
    rng = np.random.default_rng(seed)
    oa, ob = rng.standard_normal((2, Nq, H * d))
    la, lb = rng.standard_normal((2, Nq, H)) * 3
    la[0, :] = -np.inf
    lb[1, 0] = -np.inf
    return oa, la, ob, lb


@pytest.mark.parametrize("d", [6, 2, 5])
def test_lse_merge_odd_head_dim(d):
    Nq, H = 29, 3
    oa, la, ob, lb = _merge_inputs(Nq, H, d)
    ro, rl = oracle.lse_merge([(oa, la), (ob, lb)], H, d)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    for dt, tol in ((torch.float32, 1e-6), (torch.bfloat16, 8e-3)):
        out, lse = lib.lse_merge(H, d, dev(oa), dev(la), dev(ob), dev(lb), out_dtype=dt)
        torch.cuda.synchronize()
        out, lse = from_dev(out), from_dev(lse)
        log(f"merge d={d} {dt}: max err {np.max(np.abs(out - ro)):.3e}")
        assert np.max(np.abs(out - ro)) <= tol * np.max(np.abs(ro))
        fin = np.isfinite(rl)
        assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
        assert np.max(np.abs(lse[fin] - rl[fin])) < 1e-5


@pytest.mark.parametrize("which", ["a", "b"])
def test_lse_merge_in_place_f32(which):
    Nq, H, d = 37, 3, 128
    oa, la, ob, lb = _merge_inputs(Nq, H, d, seed=4)
    ro, rl = oracle.lse_merge([(oa, la), (ob, lb)], H, d)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    ta, tla, tb, tlb = dev(oa), dev(la), dev(ob), dev(lb)
    out, lout = (ta, tla) if which == "a" else (tb, tlb)
    lib.nkv_lse_merge(H, d, ta, tla, tb, tlb, out, lout)
    torch.cuda.synchronize()
    o, l_ = from_dev(out), from_dev(lout)
    assert np.max(np.abs(o - ro)) <= 1e-6 * np.max(np.abs(ro))
    fin = np.isfinite(rl)
    assert np.max(np.abs(l_[fin] - rl[fin])) < 1e-5


# --------------------------------------------------------------------------
# nearest center: duplicates and near-ties
# --------------------------------------------------------------------------

def _bf16_away_from_zero(x, floor=2.0 ** -6):
    """bf16 bits of x with |x| >= floor: every product of two such values is a
    multiple of 2^-26, so the fp64 sums of the oracle (and of an exact
    reference) have no rounding at these sizes."""
    x = np.where(np.abs(x) < floor, np.copysign(floor, x), x)
    return synth.f64_to_bf16_bits(x)


def _near_tie_set(W, A, N, seed, group=2):
    """Centers in groups of `group`: center g j + k (k >= 1) is center g j with
    one channel moved by one bf16 step (groups with j % 4 == 3: exact
    duplicates); tokens sit near the first center of a group, so the group's
    distances differ by ~3e-3 against fp32 rounding errors of ~1e-2 in
    distances near ||mu||^2 ~ 64 W.  Pairs leave a 64-center slot's third
    nearest far away (two candidates per slot); triples bring the third
    within the bound too (the whole slot is searched).  Centers past the
    last whole group are independent draws."""
    rng = np.random.default_rng(seed)
    ng = A // group
    base = _bf16_away_from_zero(8.0 * rng.standard_normal((A, W)))
    mu = base.copy()
    for j in range(ng):
        for k in range(1, group):
            mu[group * j + k] = mu[group * j]
            if j % 4 != 3:
                c = rng.integers(0, W)
                mu[group * j + k, c] = np.uint16(int(mu[group * j, c]) +
                                                 (1 if rng.random() < 0.5 else -1))
    a = rng.integers(0, ng, size=N) * group
    x = synth.bf16_bits_to_f64(mu[a]) + 0.05 * rng.standard_normal((N, W))
    return mu, _bf16_away_from_zero(x)


def _exact_argmin(x_bits, mu_bits, rows):
    """Exact squared-L2 argmin (ties to the lowest index) with rational
    arithmetic for a few tokens: the reference the fp64 oracle must equal."""
    out = []
    mu = [[fractions.Fraction(float(v)) for v in synth.bf16_bits_to_f64(r)] for r in mu_bits]
    for t in rows:
        x = [fractions.Fraction(float(v)) for v in synth.bf16_bits_to_f64(x_bits[t])]
        d = [sum((xi - mi) ** 2 for xi, mi in zip(x, m)) for m in mu]
        out.append(min(range(len(d)), key=lambda a: (d[a], a)))
    return np.array(out)


# (A, N): 600 tokens x 64 centers make too few 128 x 128 tiles for the chip,
# so the tuned distance product is split over K; 16384 x 256 fill it and take
# the unsplit product with its own epilogue
@pytest.mark.parametrize("group", [2, 3], ids=["pairs", "triples"])
@pytest.mark.parametrize("size", [(64, 600), (256, 16384)], ids=["split-k", "one-pass"])
@pytest.mark.parametrize("generic", [False, True])
def test_assign_near_ties_and_duplicates(generic, size, group):
    H, d, r = 2, 128, 64
    A, N = size
    W = H * d
    mu, x = _near_tie_set(W, A, N, seed=7, group=group)
    enc = synth.f64_to_bf16_bits(np.linalg.qr(np.random.default_rng(8).standard_normal((W, r)))[0].T
                                 .copy())
    ref = oracle.encode(x, mu, enc, 32, "bf16")
    # the oracle's fp64 argmin is the exact one here (spot check with rationals)
    spot = np.arange(0, N, max(75, N // 8))
    assert np.array_equal(ref["idx"][spot], _exact_argmin(x, mu, spot))
    xf = oracle.as_f64(x, "bf16")
    muf = oracle.as_f64(mu, "bf16")
    # squared distances, blockwise (exact enough here to count near ties)
    dist = np.concatenate([np.sum(xb * xb, axis=1)[:, None] + np.sum(muf * muf, axis=1)[None]
                           - 2.0 * (xb @ muf.T) for xb in np.array_split(xf, max(1, N // 2048))])
    srt = np.sort(dist, axis=1)
    close = int(np.sum(srt[:, 1] - srt[:, 0] < 1e-2))
    dup = int(np.sum(srt[:, 1] == srt[:, 0]))
    log(f"near-tie set: {N} tokens, {close} with a runner-up within 1e-2, {dup} exact ties")
    assert close > N // 2 and dup > 0
    shape = lib.Shape(H, d, r, 32, "bf16")
    lib.nkv_force_generic(generic)
    try:
        idx, codes, sc = lib.encode(shape, to_dev(x, "bf16"), to_dev(mu, "bf16"),
                                    to_dev(enc, "bf16"))
        torch.cuda.synchronize()
    finally:
        lib.nkv_force_generic(False)
    gidx = idx.cpu().numpy()
    bad = np.flatnonzero(gidx != ref["idx"])
    log(f"  generic={generic}: {len(bad)} index differences")
    assert len(bad) == 0, f"indices differ at {bad[:10]}"
    rep = check_encode(gidx, codes.cpu().numpy(), sc.cpu().numpy(), ref, 32)
    log(f"  {rep}")


@pytest.mark.parametrize("group", [2, 3], ids=["pairs", "triples"])
def test_assign_near_ties_many_tiles(group):
    """2048 centers x 32768 tokens: 16 x 256 tiles of 128 x 128, so the
    distance product's block order forms four groups of four center tiles,
    each served by two XCDs (the C4-sized fitting has two groups of four)."""
    H, d, r = 2, 128, 64
    A, N = 2048, 32768
    W = H * d
    mu, x = _near_tie_set(W, A, N, seed=11, group=group)
    enc = synth.f64_to_bf16_bits(np.linalg.qr(np.random.default_rng(8).standard_normal((W, r)))[0].T
                                 .copy())
    ref = oracle.encode(x, mu, enc, 32, "bf16")
    shape = lib.Shape(H, d, r, 32, "bf16")
    idx, codes, sc = lib.encode(shape, to_dev(x, "bf16"), to_dev(mu, "bf16"), to_dev(enc, "bf16"))
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    bad = np.flatnonzero(gidx != ref["idx"])
    log(f"many-tile near-tie set ({group} per group): {len(bad)} index differences of {N}")
    assert len(bad) == 0, f"indices differ at {bad[:10]}"
    rep = check_encode(gidx, codes.cpu().numpy(), sc.cpu().numpy(), ref, 32)
    log(f"  {rep}")


# --------------------------------------------------------------------------
# low-dimensional rows recomputed exactly (score bound too loose)
# --------------------------------------------------------------------------

def test_low_rows_with_loose_bound_take_exact_path():
    """Rows whose bound gap 2 c |q~| max|c^K| exceeds 60 (log2 units; c the
    softmax scale in log2 units) are listed by the bound kernel and
    recomputed by the exact two-pass kernel.  Scaling a few query rows by 120
    puts them past that limit; all rows must still match the oracle.

    The whole history is routed low-dimensionally: at these query sizes
    (scores of several hundred nats) a full-dimensional read over bf16
    decoded keys carries score errors of ~2^-9 |q| |k| ~ 1 nat, the
    precision of any bf16 attention, not of this path.  The current chunk's
    keys are exact bf16 inputs, so its flash part stays exact here."""
    cfg = synth.small_config("C3", H=3, r=96, A=70, n_hist=1500, Nq=150, N_cur=90, chunk=500,
                             r_low=32, n_full_tail=0, seed=61)
    case = get_case(cfg)
    w = case.w
    qf = oracle.as_f64(w.queries(), cfg.dtype)
    big = np.array([0, 7, 64, 131, 149])
    qf[big] *= 120.0
    q_bits = synth.f64_to_bf16_bits(qf)
    qf = oracle.as_f64(q_bits, cfg.dtype)
    # the kernels' criterion, evaluated here for the scaled rows
    kb_o, vb_o = oracle_branch(case, 0), oracle_branch(case, 1)
    low = np.arange(0, cfg.n_attend)
    ck = kb_o.rows(low).coefficients()[:, :cfg.r_low]
    cmax = np.sqrt(np.max(np.sum(ck * ck, axis=1)))
    D = oracle.as_f64(w.decoder(0), cfg.dtype)
    c = cfg.tau / np.log(2.0)
    gaps = []
    for h in range(cfg.H):
        qt = qf[:, h * cfg.d:(h + 1) * cfg.d] @ D[h * cfg.d:(h + 1) * cfg.d, :cfg.r_low]
        gaps.append(2 * c * np.linalg.norm(qt, axis=1) * cmax)
    gaps = np.stack(gaps, 1)
    log(f"bound gaps: scaled rows min {gaps[big].min():.1f}, others max "
        f"{np.delete(gaps, big, 0).max():.1f} (limit 60)")
    assert gaps[big].min() > 60 and np.delete(gaps, big, 0).max() < 60
    shape = shape_of(cfg)
    kb, vb = device_branch(case, 0), device_branch(case, 1)
    q = to_dev(q_bits, cfg.dtype)
    ckd, cvd = to_dev(w.current(0), cfg.dtype), to_dev(w.current(1), cfg.dtype)
    out, lse = lib.attend_fast(shape, kb, vb, cfg.n_attend, cfg.segments(), cfg.r_low, q, ckd, cvd)
    torch.cuda.synchronize()
    kf, vf = oracle.as_f64(w.current(0), cfg.dtype), oracle.as_f64(w.current(1), cfg.dtype)
    ro, rl = oracle.attend_fast(qf, kb_o, vb_o, cfg.segments(), cfg.r_low, kf, vf, cfg.H, cfg.d,
                                cfg.tau)
    o, l_ = from_dev(out), from_dev(lse)
    rel, lerr = attention_errors(o, l_, ro, rl)
    rel_b, lerr_b = attention_errors(o[big], l_[big], ro[big], rl[big])
    log(f"  all rows rel={rel:.3e} dLSE={lerr:.3e}; scaled rows rel={rel_b:.3e} dLSE={lerr_b:.3e}")
    assert rel <= OUT_TOL and lerr <= LSE_TOL and rel_b <= OUT_TOL


# --------------------------------------------------------------------------
# the generic kernels on the full C2 workload
# --------------------------------------------------------------------------

def test_generic_kernels_full_C2():
    cfg = synth.CONFIGS["C2"]
    case = get_case(cfg)
    shape = shape_of(cfg)
    kb, vb = device_branch(case, 0), device_branch(case, 1)
    q = to_dev(case.w.queries(), cfg.dtype)
    ck, cv = to_dev(case.w.current(0), cfg.dtype), to_dev(case.w.current(1), cfg.dtype)
    lib.nkv_force_generic(True)
    try:
        out, lse = lib.attend_fast(shape, kb, vb, cfg.n_attend, cfg.segments(), cfg.r_low, q, ck,
                                   cv)
        torch.cuda.synchronize()
    finally:
        lib.nkv_force_generic(False)
    rows = q_rows(cfg, 40)
    qo, cko, cvo = oracle_inputs(case, rows)
    ro, rl = oracle.attend_fast(qo, oracle_branch(case, 0), oracle_branch(case, 1),
                                cfg.segments(), cfg.r_low, cko, cvo, cfg.H, cfg.d, cfg.tau)
    rel, lerr = attention_errors(from_dev(out)[rows], from_dev(lse)[rows], ro, rl)
    log(f"generic C2: rows={len(rows)} rel={rel:.3e} dLSE={lerr:.3e}")
    assert rel <= OUT_TOL and lerr <= LSE_TOL
