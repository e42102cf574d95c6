"""The allocation-free entry point gdn_chunk_bidir_noalloc against gdn_chunk_bidir on a handle.

Both run the same kernels on the same inputs and differ only in where the workspace lives (the
library's static scratch array against the handle's allocation) and in how the items are spaced
in it, so their outputs must agree bit for bit.  Two calls in a row share the one scratch array,
the second with a smaller input (fewer items, a different sub-chunk), so a stale item left by the
first call would show up in the second.  The first call is also held to the oracle at the path's
tolerance.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import assert_close, dev_inputs, empty_out

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402


def _handle_bidir(d, D, T, C, state0):
    """gdn_chunk_bidir on a fresh handle, not committing: (o_fwd, o_rev, final forward state)."""
    B, H = d["q"].shape[0], d["q"].shape[2]
    s = gb.Stream(B, H, D, D, T, subchunk=C)
    try:
        s.state_set(state0)
        t = dev_inputs(d)
        o_f, o_r = empty_out(t), empty_out(t)
        S = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
        s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r, flags=gb.GDN_NO_COMMIT, state_out=S)
        torch.cuda.synchronize()
        return o_f, o_r, S
    finally:
        s.close()


def _noalloc_bidir(d, C, state_in, state_out, status):
    t = dev_inputs(d)
    o_f, o_r = empty_out(t), empty_out(t)
    # fill the outputs with NaN so that an element the call does not write shows up
    o_f.fill_(float("nan"))
    o_r.fill_(float("nan"))
    gb.gdn_chunk_bidir_noalloc(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r, status, subchunk=C,
                               state_in=state_in, state_out=state_out)
    torch.cuda.synchronize()
    return o_f, o_r


def _check_equal(name, x, y):
    assert torch.isfinite(x).all(), f"{name}: non-finite values"
    assert torch.equal(x, y), f"{name}: max |diff| {float((x.float() - y.float()).abs().max()):.3e}"


def test_noalloc_matches_handle_on_two_calls():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    # call 1: the 720p chunk of one GDN layer (B=1, H=20, d=112, T=2640, C=64): 22.4 MB of items
    print("noalloc call 1: B=1 H=20 D=112 T=2640 C=64 seed 71", flush=True)
    d1 = gdn_inputs.batch(71, 1, 2640, 20, 112, with_state=True)
    S0 = torch.from_numpy(d1["S0"]).cuda()
    ref1 = _handle_bidir(d1, 112, 2640, 64, S0)
    S1 = torch.full_like(S0, float("nan"))
    o_f1, o_r1 = _noalloc_bidir(d1, 64, S0, S1, status)
    assert int(status.item()) == 0
    for name, x, y in zip(("o_fwd", "o_rev", "state"), (o_f1, o_r1, S1), ref1):
        _check_equal(name, x, y)
    of, Sf = oracle.forward(d1["q"], d1["k"], d1["v"], d1["a"], d1["beta"], d1["S0"])
    orv, _ = oracle.reverse(d1["q"], d1["k"], d1["v"], d1["a"], d1["beta"])
    assert_close("o_fwd vs oracle", o_f1, of)
    assert_close("o_rev vs oracle", o_r1, orv)
    assert_close("state vs oracle", S1, Sf)

    # call 2: smaller (B=2, H=3, T=700 with a ragged last sub-chunk, C=32), the state updated in place
    print("noalloc call 2: B=2 H=3 D=112 T=700 C=32 seed 72, in-place state", flush=True)
    d2 = gdn_inputs.batch(72, 2, 700, 3, 112, with_state=True)
    S0b = torch.from_numpy(d2["S0"]).cuda()
    ref2 = _handle_bidir(d2, 112, 700, 32, S0b)
    S_inplace = S0b.clone()
    o_f2, o_r2 = _noalloc_bidir(d2, 32, S_inplace, S_inplace, status)
    assert int(status.item()) == 0
    for name, x, y in zip(("o_fwd", "o_rev", "state"), (o_f2, o_r2, S_inplace), ref2):
        _check_equal(name, x, y)


def test_noalloc_zero_state_and_empty_call():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    print("noalloc: B=1 H=2 D=64 T=200 C=64 seed 73, zero start state", flush=True)
    d = gdn_inputs.batch(73, 1, 200, 2, 64)
    zero = torch.zeros((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    ref = _handle_bidir(d, 64, 200, 64, zero)
    S = torch.empty_like(zero)
    o_f, o_r = _noalloc_bidir(d, 64, None, S, status)
    for name, x, y in zip(("o_fwd", "o_rev", "state"), (o_f, o_r, S), ref):
        _check_equal(name, x, y)
    # T = 0 copies state_in to state_out and touches nothing else
    x = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((1, 0, 2), dtype=torch.float32, device="cuda")
    dst = torch.full_like(S, float("nan"))
    gb.gdn_chunk_bidir_noalloc(x, x, x, g, g, torch.empty_like(x), torch.empty_like(x), status,
                               state_in=S, state_out=dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, S)
    assert int(status.item()) == 0


def test_noalloc_rejects_a_call_beyond_the_scratch():
    """B=1, H=20, d=112, T=8200 needs 2*20*129*13312 bytes > 64 MiB: refused, outputs untouched."""
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.zeros((1, 8200, 20, 112), dtype=torch.bfloat16, device="cuda")
    g = torch.full((1, 8200, 20), 0.5, dtype=torch.float32, device="cuda")
    o = torch.full_like(q, 3.0)
    o_r = torch.full_like(q, 3.0)
    with pytest.raises(gb.GdnError) as ei:
        gb.gdn_chunk_bidir_noalloc(q, q, q, g, g, o, o_r, status)
    assert ei.value.code == gb.GDN_E_SHAPE
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((o_r == 3.0).all())
    assert np.asarray(status.cpu())[0] == 0
