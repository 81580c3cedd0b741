"""The seeded generator: storage rounding and workload structure."""
import numpy as np
import torch

from compressed_history_attention_amd import synth


def test_bf16_round_half_even_hand_cases():
    one = 0x3F80
    cases = {
        1.0: one,
        1.0 + 2.0 ** -8: one,                  # midpoint 1 | 1+2^-7 -> even (1)
        1.0 + 3 * 2.0 ** -8: one + 2,          # midpoint 1+2^-7 | 1+2^-6 -> even
        1.0 + 2.0 ** -8 + 2.0 ** -30: one + 1,  # just above the midpoint
        -2.0: 0xC000,
        0.0: 0x0000,
    }
    xs = np.array(list(cases.keys()))
    got = synth.f64_to_bf16_bits(xs)
    assert got.tolist() == list(cases.values())


def test_bf16_matches_torch_away_from_midpoints():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))
    x32 = x.astype(np.float32).astype(np.float64)   # fp32 values: torch rounds fp32->bf16 once
    ours = synth.f64_to_bf16_bits(x32)
    ref = torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_workload_shapes_and_determinism():
    w1, w2 = synth.workload("C0"), synth.workload("C0")
    assert np.array_equal(w1.queries(), w2.queries())
    x, a, z = w1.history_chunk(0, 0)
    c = w1.cfg
    assert x.shape == (c.n_hist, c.W) and a.shape == (c.n_hist,) and z.shape == (c.n_hist, c.r)
    assert w1.encoder(0).shape == (c.r, c.W)
    assert np.array_equal(w1.encoder(1), w1.decoder(1).T)


def test_routing_policies():
    c2, c3, c4 = (synth.CONFIGS[n] for n in ("C2", "C3", "C4"))
    assert c2.segments() == [(0, 3 * 4680, 1), (3 * 4680, 4 * 4680, 0)]
    assert c3.segments() == [(0, 10 * 4680, 1), (10 * 4680, 12 * 4680, 0)]
    assert c4.n_attend == 33 * 4680
    assert c4.segments() == [(0, 29 * 4680, 1), (29 * 4680, 33 * 4680, 0)]
