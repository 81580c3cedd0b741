"""GPU parity of center fitting (nkv_fit_centers: Lloyd iterations; the
pages fit K and V centers per branch, Table 5 caption) against the fp64
oracle.  Bars: assignments bit-exact, fitted centers bit-exact (one
round-half-to-even of the mean to the storage dtype on both sides), counts
exact; empty centers keep their values; no rows leaves the centers alone.
"""
import numpy as np
import pytest
import torch

from compressed_history_attention_amd import lib, synth
from gpu_cases import log, to_dev
from oracle import fit

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    yield
    torch.cuda.synchronize()


def _from_dev(t, dtype):
    a = t.cpu()
    if dtype == "bf16":
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def _init_from_labels(x, labels, A, rng):
    """One row of every generating cluster (a sensible k-means start)."""
    rows = [rng.choice(np.flatnonzero(labels == a)) for a in range(A) if (labels == a).any()]
    return x[np.array(rows)]


def _check(cfg, x, mu0, iters):
    shape = lib.Shape(cfg.H, cfg.d, cfg.r, cfg.group, cfg.dtype)
    cd = to_dev(mu0, cfg.dtype).contiguous()
    xd = to_dev(x, cfg.dtype)
    log(f"fit {cfg.dtype} N={x.shape[0]} W={cfg.W} A={mu0.shape[0]} iters={iters}")
    c, idx, cnt = lib.fit_centers(shape, xd, cd, iters)
    torch.cuda.synchronize()
    rc, ridx, rcnt = fit.lloyd(x, mu0, iters, cfg.dtype)
    gc = _from_dev(c, cfg.dtype)
    diff = np.argwhere(gc != rc)
    assert diff.size == 0, f"{len(diff)} center values differ, first {diff[:5]}"
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    log(f"  centers moved: {int((rc != mu0).any(axis=1).sum())} of {mu0.shape[0]}")


def test_fit_tuned_from_label_rows():
    cfg = synth.small_config("C3", H=4, r=128, A=64, n_hist=3000, chunk=3000)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(0, 0)
    mu0 = _init_from_labels(x, labels, cfg.A, np.random.default_rng(1))
    for iters in (0, 1, 3):
        _check(cfg, x, mu0, iters)


def test_fit_tuned_random_row_start():
    """Centers started from random rows, as a k-means++-free start does:
    several rows of one generating cluster become near-duplicate centers,
    so many tokens sit within the assignment's rounding bound of two or
    three of them and are assigned again exactly; results still bit-exact."""
    cfg = synth.small_config("C3", H=4, r=128, A=64, n_hist=3000, chunk=3000)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(0, 0)
    rng = np.random.default_rng(5)
    sel = rng.choice(x.shape[0], cfg.A, replace=False)
    mu0 = x[sel]
    multi = int((np.bincount(labels[sel], minlength=cfg.A) >= 2).sum())
    log(f"random-row start: {multi} generating clusters hold two or more starting centers")
    assert multi > 0
    for iters in (1, 3):
        _check(cfg, x, mu0, iters)


def test_fit_tuned_perturbed_centers_with_empty_cluster():
    cfg = synth.small_config("C3", H=4, r=128, A=64, n_hist=2000, chunk=2000)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(1, 0)
    rng = np.random.default_rng(2)
    mu = synth.bf16_bits_to_f64(w.centers(1)) + 0.05 * rng.standard_normal((cfg.A, cfg.W))
    mu[7] += 100.0    # far away: receives no rows and must keep its value
    mu0 = synth.f64_to_bf16_bits(mu)
    _check(cfg, x, mu0, 2)


def test_fit_generic_f32():
    cfg = synth.small_config("C3", H=2, d=64, r=32, A=16, group=16, dtype="f32", n_hist=900,
                             chunk=900)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(0, 0)
    mu0 = _init_from_labels(x, labels, cfg.A, np.random.default_rng(3))
    _check(cfg, x, mu0, 2)


def test_fit_tuned_ragged_counts():
    # center count not a multiple of the 64-row LDS blocks, rows not a
    # multiple of anything
    cfg = synth.small_config("C3", H=4, r=128, A=100, n_hist=777, chunk=777)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(0, 0)
    mu0 = _init_from_labels(x, labels, cfg.A, np.random.default_rng(4))
    _check(cfg, x, mu0, 2)


def test_fit_no_rows():
    cfg = synth.small_config("C3", H=4, r=128, A=64)
    shape = lib.Shape(cfg.H, cfg.d, cfg.r, cfg.group, cfg.dtype)
    mu0 = synth.workload(cfg).centers(0)
    cd = to_dev(mu0, cfg.dtype).contiguous()
    x = torch.empty((0, cfg.W), dtype=torch.bfloat16, device="cuda")
    c, _, cnt = lib.fit_centers(shape, x, cd, 3)
    torch.cuda.synchronize()
    assert np.array_equal(_from_dev(c, cfg.dtype), mu0)
    assert not cnt.cpu().numpy().any()
