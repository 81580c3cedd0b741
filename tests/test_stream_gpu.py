"""Stream semantics of the Fast read.

Every kernel of a call runs on the caller's stream (the library creates no
streams or events of its own): the result must be complete once that stream
is, whichever stream it is, and the call must capture into a HIP graph whose
replays reproduce the eager result.  Both the per-head-width call (several
low-dimensional passes) and the one-width call are checked.
"""
import pytest
import torch

from compressed_history_attention_amd import lib, synth
from gpu_cases import device_branch, get_case, log, shape_of, to_dev

pytestmark = pytest.mark.gpu

CFG = synth.small_config("C3", H=3, r=96, A=70, n_hist=1500, Nq=150, N_cur=90, chunk=500,
                         r_low=32, n_full_tail=333, seed=51)


@pytest.fixture(scope="module")
def inputs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()
    case = get_case(CFG)
    kb, vb = device_branch(case, 0), device_branch(case, 1)
    q = to_dev(case.w.queries(), CFG.dtype)
    ck = to_dev(case.w.current(0), CFG.dtype)
    cv = to_dev(case.w.current(1), CFG.dtype)
    return (shape_of(CFG), kb, vb, CFG.n_attend, CFG.segments(), CFG.r_low, q, ck, cv)


WIDTHS = {"per_head": [32, 48, 16], "uniform": 32}


def _read(args, widths):
    shape, kb, vb, n, route, _, q, ck, cv = args
    return lib.attend_fast(shape, kb, vb, n, route, widths, q, ck, cv)


@pytest.mark.parametrize("kind", ["per_head", "uniform"])
def test_fast_read_on_another_stream(inputs, kind):
    widths = WIDTHS[kind]
    ref_out, ref_lse = _read(inputs, widths)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, lse = _read(inputs, widths)
    s.synchronize()  # the caller's stream alone
    log(f"stream read {kind}: Nq={CFG.Nq} out equal={torch.equal(out, ref_out)}")
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


@pytest.mark.parametrize("kind", ["per_head", "uniform"])
def test_fast_read_graph_replays(inputs, kind):
    widths = WIDTHS[kind]
    ref_out, ref_lse = _read(inputs, widths)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _read(inputs, widths)  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out, lse = _read(inputs, widths)
    torch.cuda.synchronize()
    for i in range(3):
        # eager work between replays, and outputs poisoned before each
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {kind} {i}: junk={float(junk):.3f} equal={torch.equal(out, ref_out)}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
