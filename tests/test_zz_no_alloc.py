"""nkv_encode_noalloc: the encoder with the library's fixed device scratch
instead of a caller workspace, checked against nkv_encode through the C ABI
(the same kernels: results equal bit for bit, and equal to the oracle's
encoding by the encoder's parity rules) on two calls in a row, the second
with fewer tokens, and refused sizes before any device work."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from compressed_history_attention_amd import lib, synth
from gpu_cases import check_encode, log, to_dev


def test_noalloc_refuses_oversize_on_host():
    """A call whose scratch would not fit is refused before the device is
    touched (runs without a GPU too)."""
    L = lib.load()
    sh = lib.nkv_shape(24, 128, 384, 32, 1, 0.0)
    n_big = 20000
    need = L.nkv_encode_workspace_size(ctypes.byref(sh), n_big, 1024)
    assert need > lib.NOALLOC_SCRATCH_BYTES
    FAKE = 0x1000
    rc = L.nkv_encode_noalloc(ctypes.byref(sh), FAKE, n_big, FAKE, 1024, FAKE, FAKE, FAKE, FAKE,
                              None)
    assert rc == 2, L.nkv_last_error()
    assert b"scratch" in L.nkv_last_error()
    # invalid shapes keep nkv_encode's own status
    bad = lib.nkv_shape(24, 100, 384, 32, 1, 0.0)
    assert L.nkv_encode_noalloc(ctypes.byref(bad), FAKE, 10, FAKE, 1024, FAKE, FAKE, FAKE, FAKE,
                                None) == 2


@pytest.mark.gpu
def test_noalloc_encode_matches_workspace_encode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    cfg = synth.CONFIGS["C4"]
    w = synth.workload(cfg)
    shape = lib.Shape(cfg.H, cfg.d, cfg.r, cfg.group, cfg.dtype)
    for b, n in ((0, cfg.n_new), (1, 1500)):   # two calls, the second smaller
        x = w.new_chunk(b)[0][:n]
        xd = to_dev(x, cfg.dtype)
        mu, enc = to_dev(w.centers(b), cfg.dtype), to_dev(w.encoder(b), cfg.dtype)
        ref_dev = lib.encode(shape, xd, mu, enc)
        out = (torch.full((n,), -1, dtype=torch.int32, device="cuda"),
               torch.zeros((n, cfg.r // 2), dtype=torch.uint8, device="cuda"),
               torch.zeros((n, cfg.r // cfg.group), dtype=torch.int16, device="cuda"))
        log(f"noalloc encode branch {b}: N={n}")
        lib.nkv_encode_noalloc(shape, xd, mu, enc, *out)
        torch.cuda.synchronize()
        for a, r_ in zip(out, ref_dev):
            assert torch.equal(a, r_)
        ref = oracle.encode(x, w.centers(b), w.encoder(b), cfg.group, cfg.dtype)
        rep = check_encode(out[0].cpu().numpy(), out[1].cpu().numpy(), out[2].cpu().numpy(), ref,
                           cfg.group)
        log(f"  {rep}")
