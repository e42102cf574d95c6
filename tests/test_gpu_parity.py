"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every comparison is element by element over the whole output of a call
(o for each direction) and the whole final state, at the tolerance fixed for
this path (max-abs 2e-2, relative Frobenius 5e-3).  Inputs come from the seeded
generator; expected values only from the oracle.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import assert_close, dev_inputs, empty_out

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402


def _run_pair(d, D, T, *, C=0, flags=0, io="bf16", layout="bthd", state=True, bidir=False):
    B, H = d["q"].shape[0], d["q"].shape[2]
    # NaN-filled workspace: a read of a workspace byte the kernels did not write shows up
    s = gb.Stream(B, H, D, D, max(T, 1), subchunk=C, io_dtype=io, poison_ws=True)
    try:
        if state:
            s.state_set(torch.from_numpy(d["S0"]).cuda())
        t = dev_inputs(d, io=io, layout=layout)
        o_f, o_r = empty_out(t), empty_out(t)
        if bidir:
            s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r, flags=flags)
        else:
            s.forward(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, flags=flags)
            s.reverse(t["q"], t["k"], t["v"], t["a"], t["beta"], o_r, flags=flags)
        S = s.state_get()
        torch.cuda.synchronize()
        return o_f, o_r, S
    finally:
        s.close()


def _oracle_pair(d, state=True):
    S0 = d["S0"] if state else None
    of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S0)
    orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"])
    return of, orv, Sf


def test_720p_chunk_forward_and_reverse_chunked():
    """One GDN layer, one 720p chunk: B=1, H=20, d=112, T=2640, carried N(0, 0.1) state."""
    d = gdn_inputs.batch(1, 1, 2640, 20, 112, with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, 112, 2640)
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


def test_720p_chunk_sequential_kernel():
    d = gdn_inputs.batch(1, 1, 2640, 20, 112, with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, 112, 2640, flags=gb.GDN_SEQUENTIAL)
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf, rel_f=1e-4)


@pytest.mark.parametrize("D", [16, 32, 64, 112, 128])
@pytest.mark.parametrize("C", [16, 32, 64])
def test_small_shapes_chunked(D, C):
    """Several sub-chunks plus a ragged tail (77 tokens), two streams, three heads."""
    d = gdn_inputs.batch(50 + D, 2, 77, 3, D, with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, D, 77, C=C)
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


@pytest.mark.parametrize("T", [1, 15, 16, 63, 64, 65, 128, 129])
def test_sequence_length_edges(T):
    d = gdn_inputs.batch(60, 1, T, 2, 112, with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, 112, T)
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


def test_tiny_fp32_sequential():
    """B=1, H=1, d=16, T=64, fp32, zero initial state, seed 0 (token-sequential kernel)."""
    d = gdn_inputs.tiny_fp32()
    of, orv, Sf = _oracle_pair(d, state=False)
    o_f, o_r, S = _run_pair(d, 16, 64, io="f32", state=False, flags=gb.GDN_SEQUENTIAL)
    assert_close("o_fwd", o_f, of, rel_f=1e-5)
    assert_close("o_rev", o_r, orv, rel_f=1e-5)
    assert_close("state", S, Sf, rel_f=1e-5)


def test_tiny_fp32_chunked():
    """The tiny configuration (B=1, H=1, d=16, T=64, sub-chunk 16, fp32, zero initial state,
    seed 0) through the chunked kernels: q, k, v are staged as bf16, o is stored in fp32."""
    d = gdn_inputs.tiny_fp32()
    of, orv, Sf = _oracle_pair(d, state=False)
    o_f, o_r, S = _run_pair(d, 16, 64, C=16, io="f32", state=False)
    assert o_f.dtype == torch.float32
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


@pytest.mark.parametrize("C", [16, 64])
def test_fp32_io_chunked(C):
    """fp32 I/O through the chunked kernels at d = 112 with a carried state and a ragged tail."""
    d = gdn_inputs.batch(63, 2, 700, 3, 112, io="f32", with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, 112, 700, C=C, io="f32", bidir=True)
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_repeated_bidir_calls_are_bitwise_identical(C):
    """Fresh handles (fresh workspace memory) and the same inputs give the same bits every time:
    the kernels read nothing they have not written and reduce in a fixed order."""
    d = gdn_inputs.batch(63, 2, 700, 3, 112, io="f32", with_state=True)
    first = _run_pair(d, 112, 700, C=C, io="f32", bidir=True)
    for x in first:
        assert torch.isfinite(x).all()
    for _ in range(5):
        again = _run_pair(d, 112, 700, C=C, io="f32", bidir=True)
        for x, y in zip(first, again):
            assert torch.equal(x, y)


def test_bidir_equals_separate_calls_bitwise():
    d = gdn_inputs.batch(61, 2, 300, 4, 112, with_state=True)
    a = _run_pair(d, 112, 300)
    b = _run_pair(d, 112, 300, bidir=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_head_major_layout():
    """q/k/v/o stored [B, H, T, D] (strided views) give the same result."""
    d = gdn_inputs.batch(62, 2, 150, 3, 112, with_state=True)
    of, orv, Sf = _oracle_pair(d)
    o_f, o_r, S = _run_pair(d, 112, 150, layout="bhtd")
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)
