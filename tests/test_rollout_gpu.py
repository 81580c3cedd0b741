"""GPU parity of the multi-layer rollout driver against the oracle's chunk
loop: per-layer Table 7 routing policies (anchors + recent frames; sink +
recent after an all-full start; full-layer fallback), per-head widths
(Table 6), encode-append of every finished chunk, and the storage account
of the caches the driver really holds.

Bars as in the other parity tests: every chunk's attention output within
max|err| / max|ref| <= 1e-2 and LSE within 1e-3; appended encodings follow
the encoder parity rules (indices bit-exact, codes bit-exact outside the
rounding window).
"""
import numpy as np
import pytest
import torch

from compressed_history_attention_amd import lib, synth
from compressed_history_attention_amd.rollout import Rollout
from gpu_cases import attention_errors, check_encode, from_dev, log, to_dev
from oracle import nanokv_oracle as nk
from oracle import rollout as ro

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 1e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    yield
    torch.cuda.synchronize()


def _inputs(base, n_layers, n_chunks, chunk, Nq, seed0, **kw):
    """Per layer a seeded codec; per chunk and layer queries and K/V rows."""
    wls = [synth.workload(synth.small_config(base, seed=seed0 + l, n_hist=chunk * n_chunks,
                                             Nq=Nq, N_cur=chunk, chunk=chunk, **kw))
           for l in range(n_layers)]
    cfg = wls[0].cfg
    chunks = []
    for c in range(n_chunks):
        row = []
        for l, wl in enumerate(wls):
            rng = np.random.default_rng([seed0, 77, l, c])
            q = synth.store(rng.standard_normal((Nq, cfg.W)), cfg.dtype)
            row.append((q, wl.history_chunk(0, c)[0], wl.history_chunk(1, c)[0]))
        chunks.append(row)
    return cfg, wls, chunks


def _run(cfg, wls, chunks, policies, widths):
    shape = lib.Shape(cfg.H, cfg.d, cfg.r, cfg.group, cfg.dtype)
    dev_codecs = [((to_dev(w.centers(0), cfg.dtype), to_dev(w.centers(1), cfg.dtype)),
                   (to_dev(w.encoder(0), cfg.dtype), to_dev(w.encoder(1), cfg.dtype)),
                   (to_dev(w.decoder(0), cfg.dtype), to_dev(w.decoder(1), cfg.dtype)))
                  for w in wls]
    n_tok = sum(row[0][1].shape[0] for row in chunks)
    lib_pols = [lib.RoutePolicy(**p.__dict__) for p in policies]
    roll = Rollout(shape, dev_codecs, lib_pols, widths, capacity=n_tok + 5)
    got = []
    for c, row in enumerate(chunks):
        ins = [(to_dev(q, cfg.dtype), to_dev(k, cfg.dtype), to_dev(v, cfg.dtype))
               for q, k, v in row]
        outs = roll.chunk(ins)
        torch.cuda.synchronize()
        got.append([(from_dev(o), from_dev(l)) for o, l in outs])
        log(f"  chunk {c}: n_hist {roll.n_hist}")
    codecs = [ro.LayerCodec((w.centers(0), w.centers(1)), (w.encoder(0), w.encoder(1)),
                            (w.decoder(0), w.decoder(1))) for w in wls]
    ref = ro.rollout(codecs, policies, chunks, cfg.H, cfg.d, cfg.group, cfg.dtype, cfg.tau,
                     widths)
    worst = (0.0, 0.0)
    for c in range(len(chunks)):
        for l in range(len(wls)):
            rel, lerr = attention_errors(got[c][l][0], got[c][l][1], ref[c][l][0], ref[c][l][1])
            worst = (max(worst[0], rel), max(worst[1], lerr))
            assert rel <= OUT_TOL and lerr <= LSE_TOL, (c, l, rel, lerr)
    log(f"  worst rel {worst[0]:.2e} lse {worst[1]:.2e}")
    return roll


def _check_history(roll, cfg, wls, chunks, layer):
    """The driver's stored records equal the oracle encoding of the chunks."""
    for b in range(2):
        x = np.concatenate([row[layer][1 + b] for row in chunks])
        ref = nk.encode(x, wls[layer].centers(b), wls[layer].encoder(b), cfg.group, cfg.dtype)
        n = roll.caches[layer].n_hist
        assert n == x.shape[0]
        c = roll.caches[layer]
        check_encode(c.idx[b][:n].cpu().numpy(), c.codes[b][:n].cpu().numpy(),
                     c.scales[b][:n].cpu().numpy(), ref, cfg.group)


def _check_storage(roll, cfg):
    st = roll.storage()
    held = sum(c.history_bytes() for c in roll.caches)
    assert st["cached"] == held
    want = ro.storage(cfg.H, cfg.d, cfg.r, cfg.group, cfg.A, cfg.A, roll.n_hist,
                      2 if cfg.dtype == "bf16" else 4)
    assert st["cached"] == len(roll.caches) * want["cached"]
    assert st["resident"] == len(roll.caches) * want["resident"]
    assert st["cr_effective"] == pytest.approx(want["cr_effective"], rel=1e-12)
    log(f"  storage {st['total']} B, effective CR {st['cr_effective']:.2f}")


def test_rollout_tuned_table7_policies():
    # bf16, d = 128: the tuned kernels.  Frames of 64 tokens, chunks of three
    # frames; three layers with the three Table 7 policy families
    frame = 64
    cfg, wls, chunks = _inputs("C3", n_layers=3, n_chunks=5, chunk=3 * frame, Nq=200,
                               seed0=300, H=4, r=128, A=64)
    policies = [ro.RoutePolicy(frame_tokens=frame, recent_frames=4, anchor_every=4),
                ro.RoutePolicy(frame_tokens=frame, sink_frames=1, recent_frames=2,
                               all_full_frames=6),
                ro.RoutePolicy(frame_tokens=frame, recent_frames=4, layer_full=True)]
    widths = [[32, 64, 96, 128], 64, 48]
    log(f"rollout tuned H={cfg.H} r={cfg.r} A={cfg.A} chunks={len(chunks)}")
    roll = _run(cfg, wls, chunks, policies, widths)
    _check_history(roll, cfg, wls, chunks, layer=1)
    _check_storage(roll, cfg)


def test_rollout_generic_ragged_frames():
    # fp32, d = 64: the generic kernels; frames that do not divide the chunk
    cfg, wls, chunks = _inputs("C3", n_layers=2, n_chunks=4, chunk=50, Nq=37, seed0=400,
                               H=2, d=64, r=32, A=16, group=16, dtype="f32")
    policies = [ro.RoutePolicy(frame_tokens=30, recent_frames=1, anchor_every=3),
                ro.RoutePolicy(frame_tokens=30, sink_frames=2, recent_frames=1)]
    widths = [[8, 20], 12]
    log(f"rollout generic H={cfg.H} d={cfg.d} r={cfg.r}")
    roll = _run(cfg, wls, chunks, policies, widths)
    _check_history(roll, cfg, wls, chunks, layer=0)
    _check_storage(roll, cfg)
    # the cache is full: one more append is refused and changes nothing
    before = roll.caches[0].n_hist
    cap = roll.caches[0].capacity
    k = torch.zeros((cap - before + 1, cfg.W), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.NkvError):
        roll.append(0, k, k)
    assert roll.caches[0].n_hist == before
