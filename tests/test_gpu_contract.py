"""The C ABI's contract on a live handle, on the GPU.

- Error paths: a call with a bad argument returns its code, enqueues nothing (o and o_rev
  keep their sentinel bytes) and leaves the state cache bitwise unchanged.
- A kernel wait that gives up (forced with a tiny GDN_SPIN_LIMIT; every kernel still exits
  because every wait is bounded) is reported as GDN_E_HIP by the next call, once; a normal
  run leaves the error word at zero.
- GDN_GATE_IS_LOG: a holds log a_t; parity against the oracle fed exp of the same values,
  and the gradient da is then dL/d(log a_t) = a_t dL/da_t.
- Options off the default path: eps = 0, l2 norm off, scale != 1, on ragged lengths.
Every numeric comparison is against the fp64 oracle at the path's tolerance (max-abs 2e-2,
relative Frobenius 5e-3).  Handles are created with GDN_POISON_WS (NaN-filled workspace), so
a read of a workspace byte the kernels did not write would show up as a non-finite output.
"""
import ctypes

import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import assert_close, dev_inputs, empty_out, metrics

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402

SENTINEL = 7.0


def _live_handle(T=256, H=3, D=64):
    """A handle whose cache holds a committed non-trivial state, the inputs of a T-token call and
    sentinel-filled outputs."""
    d = gdn_inputs.batch(90, 1, T, H, D, with_state=True)
    s = gb.Stream(1, H, D, D, T, poison_ws=True)
    s.state_set(torch.from_numpy(d["S0"]).cuda())
    t = dev_inputs(d)
    o_f, o_r = empty_out(t), empty_out(t)
    s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)   # commit once: a non-trivial cache
    torch.cuda.synchronize()
    o_f.fill_(SENTINEL)
    o_r.fill_(SENTINEL)
    return s, t, o_f, o_r


def _io(t, o, **over):
    io = gb._make_io(t["q"], t["k"], t["v"], o, t["a"], t["beta"])
    for key, val in over.items():
        setattr(io, key, val)
    return io


def _call_bidir(s, io, o_rev_ptr, T, flags=0):
    lib = gb.load_library()
    return lib.gdn_chunk_bidir(ctypes.c_void_p(s.handle), ctypes.byref(io), o_rev_ptr, T, flags, None,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _call_forward(s, io, T, flags=0):
    lib = gb.load_library()
    return lib.gdn_chunk_forward(ctypes.c_void_p(s.handle), ctypes.byref(io), T, flags, None,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _bad_cases(t, o_f, o_r, T):
    """(name, expected code, call) for every argument error a live call can make."""
    mis = torch.full((1 * T * 3 * 64 + 8,), SENTINEL, dtype=torch.bfloat16, device="cuda")
    o_mis = mis[1:1 + T * 3 * 64].view(1, T, 3, 64)   # 2-byte offset: not 16-byte aligned
    cases = [
        ("T beyond max_tokens", gb.GDN_E_SHAPE, lambda s: _call_bidir(s, _io(t, o_f), ctypes.c_void_p(o_r.data_ptr()), T + 1)),
        ("negative T", gb.GDN_E_SHAPE, lambda s: _call_bidir(s, _io(t, o_f), ctypes.c_void_p(o_r.data_ptr()), -1)),
        ("unknown call flag", gb.GDN_E_INVAL, lambda s: _call_bidir(s, _io(t, o_f), ctypes.c_void_p(o_r.data_ptr()), T, 0x80)),
        ("misaligned o", gb.GDN_E_INVAL, lambda s: _call_bidir(s, _io(t, o_mis), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("misaligned o_rev", gb.GDN_E_INVAL, lambda s: _call_bidir(s, _io(t, o_f), ctypes.c_void_p(o_mis.data_ptr()), T)),
        ("NULL o_rev", gb.GDN_E_INVAL, lambda s: _call_bidir(s, _io(t, o_f), None, T)),
        ("negative token stride", gb.GDN_E_INVAL,
         lambda s: _call_bidir(s, _io(t, o_f, o_strides=gb._Strides(T * 192, -192, 64)), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("token stride not a multiple of 16 bytes", gb.GDN_E_INVAL,
         lambda s: _call_bidir(s, _io(t, o_f, q_strides=gb._Strides(T * 3 * 68, 3 * 68, 68)), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("token stride below the row width", gb.GDN_E_INVAL,
         lambda s: _call_bidir(s, _io(t, o_f, k_strides=gb._Strides(T * 32, 32, 0)), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("negative gate stride", gb.GDN_E_INVAL,
         lambda s: _call_bidir(s, _io(t, o_f, g_strides=gb._Strides(0, -3, 1)), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("NULL a", gb.GDN_E_INVAL, lambda s: _call_bidir(s, _io(t, o_f, a=None), ctypes.c_void_p(o_r.data_ptr()), T)),
        ("NULL q", gb.GDN_E_INVAL, lambda s: _call_forward(s, _io(t, o_f, q=None), T)),
        ("q row extent beyond 2 GiB", gb.GDN_E_SHAPE,
         lambda s: _call_forward(s, _io(t, o_f, q_strides=gb._Strides(0, 1 << 23, 64)), T)),
    ]
    return cases


def test_error_paths_enqueue_nothing_and_keep_the_cache():
    T = 256
    s, t, o_f, o_r = _live_handle(T)
    try:
        before = s.state_get().clone()
        torch.cuda.synchronize()
        for name, code, call in _bad_cases(t, o_f, o_r, T):
            print(f"error case: {name}", flush=True)
            rc = call(s)
            assert rc == code, f"{name}: returned {rc}, expected {code} ({gb.gdn_last_error()})"
            assert gb.gdn_last_error(), name
            torch.cuda.synchronize()
            assert bool((o_f == SENTINEL).all()) and bool((o_r == SENTINEL).all()), f"{name}: an output was written"
            assert torch.equal(s.state_get(), before), f"{name}: the cache changed"
        # o_rev with strides other than o's cannot be expressed in the C ABI (o_rev takes o's
        # strides); the binding refuses such a pair before calling it
        o_r_other = torch.empty((1, 3, T, 64), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
        with pytest.raises(ValueError):
            s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r_other)
        # after all of that the handle still works and continues from the unchanged cache
        d = gdn_inputs.batch(90, 1, T, 3, 64, with_state=True)
        S_mid = before.double().cpu().numpy()
        o_f2, o_r2 = empty_out(t), empty_out(t)
        s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f2, o_r2)
        S = s.state_get()
        torch.cuda.synchronize()
        of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S_mid)
        assert_close("o_fwd after errors", o_f2, of)
        assert_close("state after errors", S, Sf)
    finally:
        s.close()


def test_spin_give_up_is_reported_once(monkeypatch):
    """GDN_SPIN_LIMIT=1 makes the scan's waits give up at their first poll (the loads they wait
    for cannot have landed by then); every wait is bounded, so the kernels exit normally with
    outputs that are not valid.  The next call on the handle returns GDN_E_HIP and clears the
    mark; the call after it runs."""
    T, H, D = 256, 2, 64
    d = gdn_inputs.batch(91, 1, T, H, D, with_state=True)
    monkeypatch.setenv("GDN_SPIN_LIMIT", "1")
    s = gb.Stream(1, H, D, D, T)
    monkeypatch.delenv("GDN_SPIN_LIMIT")
    try:
        t = dev_inputs(d)
        o_f, o_r = empty_out(t), empty_out(t)
        print("spin limit 1: one bidir call", flush=True)
        s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
        torch.cuda.synchronize()
        with pytest.raises(gb.GdnError) as ei:
            s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
        assert ei.value.code == gb.GDN_E_HIP
        assert "gave up" in str(ei.value)
        # reported once: the handle accepts calls again
        s.state_set(None)
        torch.cuda.synchronize()
    finally:
        s.close()
    # a handle with the default limit: a normal run leaves the error word at zero
    s = gb.Stream(1, H, D, D, T)
    try:
        for _ in range(3):
            s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
        torch.cuda.synchronize()
        s.state_get()      # checks the error word
        of, _ = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"])
        s2 = gb.Stream(1, H, D, D, T)
        try:
            s2.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
            torch.cuda.synchronize()
        finally:
            s2.close()
        assert_close("o_fwd, default limit", o_f, of)
    finally:
        s.close()


@pytest.mark.parametrize("C", [16, 64])
def test_gate_is_log_forward_and_reverse(C):
    """a passed as log a_t (fp32); the oracle gets exp of the same fp32 values in fp64."""
    T, H, D = 300, 3, 112
    d = gdn_inputs.batch(92, 2, T, H, D, with_state=True)
    la = np.log(d["a"]).astype(np.float32)
    a_ref = np.exp(la.astype(np.float64))
    of, Sf = oracle.forward(d["q"], d["k"], d["v"], a_ref, d["beta"], d["S0"])
    orv, _ = oracle.reverse(d["q"], d["k"], d["v"], a_ref, d["beta"])
    s = gb.Stream(2, H, D, D, T, subchunk=C, gate_is_log=True, poison_ws=True)
    try:
        s.state_set(torch.from_numpy(d["S0"]).cuda())
        t = dev_inputs(d)
        t["a"] = torch.from_numpy(la).cuda()
        o_f, o_r = empty_out(t), empty_out(t)
        s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
        S = s.state_get()
        torch.cuda.synchronize()
    finally:
        s.close()
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


def test_gate_is_log_sequential_and_backward():
    """The token-sequential kernel and the gradient read log a_t too; da becomes dL/d(log a_t)."""
    T, H, D = 80, 2, 32
    d = gdn_inputs.batch(93, 1, T, H, D, with_state=True)
    la = np.log(d["a"]).astype(np.float32)
    a_ref = np.exp(la.astype(np.float64))
    rng = np.random.default_rng(93)
    dO = torch.from_numpy(rng.standard_normal((1, T, H, D)).astype(np.float32)).to(torch.bfloat16)
    ref = oracle.backward(d["q"], d["k"], d["v"], a_ref, d["beta"], dO.float().numpy(), d["S0"])
    of, _ = oracle.forward(d["q"], d["k"], d["v"], a_ref, d["beta"], d["S0"])
    s = gb.Stream(1, H, D, D, T, gate_is_log=True)
    try:
        t = dev_inputs(d)
        t["a"] = torch.from_numpy(la).cuda()
        S0 = torch.from_numpy(d["S0"]).cuda()
        s.state_set(S0)
        o = empty_out(t)
        s.forward(t["q"], t["k"], t["v"], t["a"], t["beta"], o, flags=gb.GDN_SEQUENTIAL)
        g = s.backward(t["q"], t["k"], t["v"], t["a"], t["beta"], dO.cuda(), state0=S0)
        torch.cuda.synchronize()
    finally:
        s.close()
    assert_close("o_fwd sequential", o, of)
    m, r = metrics(g["da"], ref["da"] * a_ref)
    print(f"  d/dlog a: max_abs={m:.3e} rel_F={r:.3e}", flush=True)
    assert r <= 2e-5
    m, r = metrics(g["dq"], ref["dq"])
    assert r <= 2e-5


@pytest.mark.parametrize("l2norm, eps, scale, T, C", [
    (True, 0.0, 1.0, 150, 64),      # eps = 0 with a ragged last sub-chunk (padded rows have zero norm)
    (True, 0.0, 0.5, 2640, 64),     # the 720p length (41 full sub-chunks + 16 tokens) at eps = 0
    (False, 1e-6, 1.0, 150, 64),    # no normalisation (inputs scaled to about unit norm)
    (False, 1e-6, 0.3, 77, 32),
    (True, 1e-3, 2.0, 45, 16),
])
def test_options_off_the_default_path(l2norm, eps, scale, T, C):
    H, D = 2, 112
    d = gdn_inputs.batch(94, 1, T, H, D, with_state=True)
    if not l2norm:
        for key in ("q", "k"):
            d[key] = gdn_inputs.round_bf16(d[key] / np.sqrt(D)).astype(np.float32)
    kw = dict(l2norm=l2norm, eps=eps, scale=scale)
    of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], **kw)
    orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"], **kw)
    s = gb.Stream(1, H, D, D, T, subchunk=C, l2norm=l2norm, l2_eps=eps, scale=scale, poison_ws=True)
    try:
        s.state_set(torch.from_numpy(d["S0"]).cuda())
        t = dev_inputs(d)
        o_f, o_r = empty_out(t), empty_out(t)
        s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r)
        S = s.state_get()
        torch.cuda.synchronize()
    finally:
        s.close()
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)
