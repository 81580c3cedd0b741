"""Pins of the center-fitting oracle (Lloyd iterations of k-means; the pages
fit centers per K/V branch, Table 5 caption, without printing the method).

* round_to_bf16 against hand-derived cases (exact ties to even, carries into
  the exponent, subnormal quantum) and against the input generator's own,
  independently written integer rounding;
* a brute-force loop version of Lloyd's method on tiny inputs;
* closed form: one iteration from the generating centers reproduces the
  generating labels and gives the per-label means;
* empty clusters keep their centers; the objective never increases (fp32).
"""
import math

import numpy as np
import pytest

from compressed_history_attention_amd import synth
from oracle import fit
from oracle import nanokv_oracle as nk


def test_round_to_bf16_hand_cases():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,            # tie -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # tie -> even (1 + 2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,  # just above the tie
        -2.0 + 2.0 ** -9: 0xC000,           # -1.998..: rounds to -2 (carry)
        2.0 ** -133: 0x0001,                # smallest bf16 subnormal
        3 * 2.0 ** -134: 0x0002,            # subnormal tie -> even
        0.0: 0x0000,
    }
    got = fit.round_to_bf16(np.array(list(cases)))
    assert [int(v) for v in got] == list(cases.values())


def test_round_to_bf16_matches_generator_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        (rng.integers(-2 ** 20, 2 ** 20, 5000) + 0.5) * 2.0 ** -12])
    assert np.array_equal(fit.round_to_bf16(x), synth.f64_to_bf16_bits(x))


def _brute_lloyd(x, mu, iters):
    x = [list(map(float, r)) for r in x]
    mu = [list(map(float, r)) for r in mu]
    A, W = len(mu), len(mu[0])

    def assign():
        out = []
        for r in x:
            best, ba = math.inf, -1
            for a in range(A):
                dd = sum((r[w] - mu[a][w]) ** 2 for w in range(W))
                if dd < best:
                    best, ba = dd, a
            out.append(ba)
        return out

    for _ in range(iters):
        lab = assign()
        for a in range(A):
            mem = [r for r, l in zip(x, lab) if l == a]
            if mem:
                mu[a] = [float(np.float32(sum(r[w] for r in mem) / len(mem))) for w in range(W)]
    return np.array(mu), assign()


def test_lloyd_brute_force_f32():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((30, 5)).astype(np.float32)
    mu0 = rng.standard_normal((4, 5)).astype(np.float32)
    for iters in (0, 1, 3):
        c, idx, cnt = fit.lloyd(x, mu0, iters, "f32")
        cb, lb = _brute_lloyd(x, mu0, iters)
        np.testing.assert_array_equal(c.astype(np.float64), cb)
        assert idx.tolist() == lb
        assert cnt.tolist() == np.bincount(lb, minlength=4).tolist()


def test_one_iteration_from_generating_centers_gives_label_means():
    cfg = synth.small_config("C3", H=2, r=32, A=16, n_hist=600, chunk=600)
    w = synth.workload(cfg)
    x, labels, _ = w.history_chunk(0, 0)
    mu0 = w.centers(0)
    c, idx, cnt = fit.lloyd(x, mu0, 1, cfg.dtype)
    xf = synth.bf16_bits_to_f64(x)
    for a in range(cfg.A):
        sel = labels == a
        if sel.any():
            want = synth.f64_to_bf16_bits(xf[sel].mean(axis=0))
            assert np.array_equal(c[a], want)
        else:
            assert np.array_equal(c[a], mu0[a])
    # the fitted centers still reproduce the labels here
    assert np.array_equal(idx, labels)
    assert cnt.tolist() == np.bincount(labels, minlength=cfg.A).tolist()


def test_empty_cluster_keeps_center_and_objective_decreases():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 8)).astype(np.float32)
    mu0 = np.concatenate([rng.standard_normal((5, 8)), np.full((1, 8), 1e3)]).astype(np.float32)
    prev = fit.objective(x, mu0, "f32")
    c = mu0
    for it in range(5):
        c, idx, cnt = fit.lloyd(x, c, 1, "f32")
        assert np.array_equal(c[5], mu0[5]) and cnt[5] == 0
        obj = fit.objective(x, c, "f32")
        assert obj <= prev * (1 + 1e-6)
        prev = obj


def test_zero_iterations_is_assignment_only():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 6)).astype(np.float32)
    mu0 = rng.standard_normal((7, 6)).astype(np.float32)
    c, idx, cnt = fit.lloyd(x, mu0, 0, "f32")
    assert np.array_equal(c, mu0)
    assert np.array_equal(idx, nk.assign_direct(x.astype(np.float64), mu0.astype(np.float64)))
