"""GPU parity of the time-split forward scan (gdn_chunk_forward_split): the whole output and the
final state of every call against the fp64 oracle's forward scan, at the path's tolerance (max-abs
2e-2, relative Frobenius 5e-3).  The split is an exact rearrangement of the same recurrence
(segment states from zero and from the identity, a serial pass over the segments, each segment
again from its start state), so the oracle of the plain scan is the reference.  Inputs come from
the seeded generator; expected values only from the oracle."""
import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import assert_close, dev_inputs, empty_out

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402


def _run_split(d, D, T, segments, *, C=0, io="bf16", flags=0, state_out=False):
    B, H = d["q"].shape[0], d["q"].shape[2]
    # NaN-filled workspace: a read of an item byte the prep did not write shows up
    s = gb.Stream(B, H, D, D, max(T, 1), subchunk=C, io_dtype=io, poison_ws=True)
    try:
        s.state_set(torch.from_numpy(d["S0"]).cuda())
        t = dev_inputs(d, io=io)
        o = empty_out(t)
        so = torch.full(s.shape, float("nan"), dtype=torch.float32, device="cuda") if state_out else None
        s.forward_split(t["q"], t["k"], t["v"], t["a"], t["beta"], o, segments, flags=flags, state_out=so)
        S = s.state_get()
        torch.cuda.synchronize()
        return o, S, so
    finally:
        s.close()


def _oracle(d):
    return oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"])


@pytest.mark.parametrize("segments", [2, 3, 7, 42, 100])
def test_720p_width_single_head(segments):
    """One stream-head of the 720p layer's width over a 2640-token chunk (42 steps of 64 tokens):
    segments of 21, 14 and 6 steps, of one step each, and more segments asked for than steps."""
    d = gdn_inputs.batch(31, 1, 2640, 1, 112, with_state=True)
    of, Sf = _oracle(d)
    o, S, _ = _run_split(d, 112, 2640, segments)
    assert_close("o", o, of)
    assert_close("state", S, Sf)


@pytest.mark.parametrize("D, C, segments", [(64, 32, 4), (112, 64, 3), (128, 16, 5), (32, 64, 2), (16, 16, 9)])
def test_small_shapes_ragged(D, C, segments):
    """Two streams, three heads, 301 tokens: a ragged last step inside the last segment."""
    d = gdn_inputs.batch(60 + D, 2, 301, 3, D, with_state=True)
    of, Sf = _oracle(d)
    o, S, _ = _run_split(d, D, 301, segments, C=C)
    assert_close("o", o, of)
    assert_close("state", S, Sf)


def test_720p_layer_all_heads():
    """The 720p chunk with all 20 heads in 3 segments (14 steps each)."""
    d = gdn_inputs.batch(32, 1, 2640, 20, 112, with_state=True)
    of, Sf = _oracle(d)
    o, S, _ = _run_split(d, 112, 2640, 3)
    assert_close("o", o, of)
    assert_close("state", S, Sf)


def test_fp32_io_and_no_commit():
    """fp32 I/O; GDN_NO_COMMIT leaves the cache at the start state and puts the final state in
    state_out."""
    d = gdn_inputs.batch(33, 1, 700, 2, 64, io="f32", with_state=True)
    of, Sf = _oracle(d)
    o, S, so = _run_split(d, 64, 700, 4, io="f32", flags=gb.GDN_NO_COMMIT, state_out=True)
    assert_close("o", o, of)
    assert_close("state_out", so, Sf)
    assert torch.equal(S.cpu(), torch.from_numpy(d["S0"]).float())


def test_repeatable_bitwise_and_close_to_the_plain_scan():
    """Two split calls on the same inputs and start state give the same bits; the plain forward
    call of the same library agrees with the split to the oracle tolerance."""
    d = gdn_inputs.batch(34, 1, 1500, 2, 112, with_state=True)
    B, H = 1, 2
    s = gb.Stream(B, H, 112, 112, 1500)
    try:
        t = dev_inputs(d)
        S0 = torch.from_numpy(d["S0"]).cuda()
        outs = []
        for _ in range(2):
            s.state_set(S0)
            o = empty_out(t)
            s.forward_split(t["q"], t["k"], t["v"], t["a"], t["beta"], o, 6, flags=gb.GDN_NO_COMMIT)
            outs.append(o)
        s.state_set(S0)
        op = empty_out(t)
        s.forward(t["q"], t["k"], t["v"], t["a"], t["beta"], op, flags=gb.GDN_NO_COMMIT)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        assert_close("split vs plain", outs[0], op.float().cpu().numpy())
    finally:
        s.close()


def test_rejected_calls_leave_the_cache_unchanged():
    d = gdn_inputs.batch(35, 1, 200, 1, 64, with_state=True)
    s = gb.Stream(1, 1, 64, 64, 200)
    try:
        S0 = torch.from_numpy(d["S0"]).cuda()
        s.state_set(S0)
        t = dev_inputs(d)
        o = torch.full_like(t["v"], 7.0)
        for segments, flags in ((0, 0), (-3, 0), (4, gb.GDN_SEQUENTIAL)):
            with pytest.raises(gb.GdnError) as ei:
                s.forward_split(t["q"], t["k"], t["v"], t["a"], t["beta"], o, segments, flags=flags)
            assert ei.value.code == gb.GDN_E_INVAL
        torch.cuda.synchronize()
        assert torch.equal(s.state_get().cpu(), S0.cpu())
        assert bool((o == 7.0).all())
    finally:
        s.close()
