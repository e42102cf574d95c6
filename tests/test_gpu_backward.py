"""GPU parity of the scan's gradient (gdn_chunk_backward, through the C ABI) against the fp64
oracle's gradient (``oracle.backward``, pinned by finite differences).

The GPU path computes in fp32 from the same input values the oracle sees (bf16-exact or
fp32), so the bar is fp32 rounding (unit roundoff 6e-8) accumulated along the scan:
relative Frobenius <= 2e-5 and max-abs <= 2e-5 of the largest reference entry, on every
gradient of a call (measured ~1e-7 to 2e-7 at up to 700 tokens)."""
import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import dev_inputs, metrics

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402

REL_F = 2e-5
MAX_REL = 2e-5


def _close(name, gpu, ref):
    m, r = metrics(gpu, ref)
    scale = float(np.abs(ref).max()) if np.size(ref) else 0.0
    print(f"  {name}: max_abs={m:.3e} (max |ref| {scale:.3e}) rel_F={r:.3e}", flush=True)
    assert r <= REL_F and m <= MAX_REL * scale + 1e-6, name


def _grads(d, D, Dv, T, *, io="bf16", reverse=False, seed=0, with_state=True, with_final=True):
    B, H = d["q"].shape[0], d["q"].shape[2]
    rng = np.random.default_rng(1000 + seed)
    dO = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    if io == "bf16":
        dO = torch.from_numpy(dO).to(torch.bfloat16).float().numpy()
    dSf = rng.standard_normal((B, H, Dv, D)).astype(np.float32) if with_final else None
    S0 = d["S0"] if (with_state and not reverse) else None
    ref = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO, S0, dSf, reverse=reverse)
    # NaN-filled workspaces: a checkpoint or partial sum read before it is written fails the test
    s = gb.Stream(B, H, D, Dv, max(T, 1), io_dtype=io, poison_ws=True)
    try:
        t = dev_inputs(d, io=io)
        dt = torch.bfloat16 if io == "bf16" else torch.float32
        g = s.backward(t["q"], t["k"], t["v"], t["a"], t["beta"], torch.from_numpy(dO).to("cuda", dt),
                       reverse=reverse,
                       d_state=None if dSf is None else torch.from_numpy(dSf).cuda(),
                       state0=None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, np.float32)).cuda())
        torch.cuda.synchronize()
    finally:
        s.close()
    return g, ref


def _check_all(g, ref):
    for key, rkey in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("da", "da"), ("dbeta", "dbeta"),
                      ("d_state0", "dS0")):
        _close(key, g[key], ref[rkey])


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("D", [16, 32, 48, 112, 128])
def test_backward_small(D, reverse):
    d = gdn_inputs.batch(70 + D, 2, 50, 3, D, with_state=True)
    g, ref = _grads(d, D, D, 50, reverse=reverse, seed=D)
    _check_all(g, ref)


def test_backward_fp32_io_and_unequal_widths():
    """fp32 q, k, v, d_o and d_k = 32 != d_v = 16."""
    rng = np.random.default_rng(5)
    B, T, H, Dk, Dv = 1, 40, 2, 32, 16
    d = {"q": rng.standard_normal((B, T, H, Dk)).astype(np.float32),
         "k": rng.standard_normal((B, T, H, Dk)).astype(np.float32),
         "v": rng.standard_normal((B, T, H, Dv)).astype(np.float32),
         "a": np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((B, T, H))))).astype(np.float32),
         "beta": (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
         "S0": (0.1 * rng.standard_normal((B, H, Dv, Dk))).astype(np.float32)}
    g, ref = _grads(d, Dk, Dv, T, io="f32", seed=5)
    _check_all(g, ref)


@pytest.mark.parametrize("D", [112, 128])
def test_backward_fp32_io_wide(D):
    """fp32 q, k, v, d_o at d = 112 and 128 (four 16-byte chunks of a staged row per lane, the
    checkpoint passes at their default occupancy), 130 tokens: two whole 64-token segments and a
    2-token tail."""
    rng = np.random.default_rng(90 + D)
    B, T, H = 1, 130, 2
    d = {"q": rng.standard_normal((B, T, H, D)).astype(np.float32),
         "k": rng.standard_normal((B, T, H, D)).astype(np.float32),
         "v": (0.5 * rng.standard_normal((B, T, H, D))).astype(np.float32),
         "a": np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((B, T, H))))).astype(np.float32),
         "beta": (1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32),
         "S0": (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)}
    g, ref = _grads(d, D, D, T, io="f32", seed=90 + D)
    _check_all(g, ref)


@pytest.mark.parametrize("reverse", [False, True])
def test_backward_720p_width_long(reverse):
    """d = 112, 700 tokens (several hundred steps of gradient flow through the state)."""
    d = gdn_inputs.batch(77, 1, 700, 2, 112, with_state=True)
    g, ref = _grads(d, 112, 112, 700, reverse=reverse, seed=77)
    _check_all(g, ref)


@pytest.mark.parametrize("reverse", [False, True])
def test_backward_720p_chunk_two_heads(reverse):
    """The benchmarked shape along time: d = 112, T = 2640 (the whole 720p chunk), 2 heads."""
    d = gdn_inputs.batch(76, 1, 2640, 2, 112, with_state=True)
    g, ref = _grads(d, 112, 112, 2640, reverse=reverse, seed=76)
    _check_all(g, ref)


def test_backward_without_final_gradient_or_start():
    d = gdn_inputs.batch(78, 1, 64, 2, 32, with_state=True)
    g, ref = _grads(d, 32, 32, 64, with_state=False, with_final=False, seed=78)
    _check_all(g, ref)


def test_backward_empty_sequence_copies_the_final_gradient():
    s = gb.Stream(1, 2, 32, 32, 16)
    try:
        q = torch.zeros((1, 0, 2, 32), dtype=torch.bfloat16, device="cuda")
        a = torch.zeros((1, 0, 2), dtype=torch.float32, device="cuda")
        dSf = torch.randn((1, 2, 32, 32), device="cuda")
        g = s.backward(q, q, q, a, a, q, d_state=dSf)
        torch.cuda.synchronize()
        assert torch.equal(g["d_state0"], dSf)
    finally:
        s.close()


def test_backward_is_bitwise_repeatable():
    d = gdn_inputs.batch(79, 1, 80, 2, 64, with_state=True)
    g1, _ = _grads(d, 64, 64, 80, seed=79)
    g2, _ = _grads(d, 64, 64, 80, seed=79)
    for key in g1:
        assert torch.equal(g1[key], g2[key]), key


def _bidir_inputs(d, D, T, seed, io="bf16"):
    B, H = d["q"].shape[0], d["q"].shape[2]
    rng = np.random.default_rng(2000 + seed)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dO = [torch.from_numpy(rng.standard_normal((B, T, H, D)).astype(np.float32)).to(dt) for _ in range(2)]
    dSf = torch.from_numpy(rng.standard_normal((B, H, D, D)).astype(np.float32))
    dSr = torch.from_numpy(rng.standard_normal((B, H, D, D)).astype(np.float32))
    return dO, dSf, dSr


def test_backward_bidir_equals_the_two_calls_bitwise():
    """gdn_chunk_backward_bidir (both scans' gradients in one launch pair) against gdn_chunk_backward
    called for each scan: the same kernels and order of operations, so the same bits.  T = 300 is
    not a multiple of the 8-token staging block."""
    B, T, H, D = 1, 300, 3, 112
    d = gdn_inputs.batch(81, B, T, H, D, with_state=True)
    dO, dSf, dSr = _bidir_inputs(d, D, T, 81)
    s = gb.Stream(B, H, D, D, T, poison_ws=True)
    try:
        t = dev_inputs(d)
        S0 = torch.from_numpy(np.ascontiguousarray(d["S0"], np.float32)).cuda()
        args = (t["q"], t["k"], t["v"], t["a"], t["beta"])
        gf, gr = s.backward_bidir(*args, dO[0].cuda(), dO[1].cuda(), d_state=dSf.cuda(), state0=S0,
                                  d_state_rev=dSr.cuda())
        ef = s.backward(*args, dO[0].cuda(), d_state=dSf.cuda(), state0=S0)
        er = s.backward(*args, dO[1].cuda(), reverse=True, d_state=dSr.cuda())
        torch.cuda.synchronize()
    finally:
        s.close()
    for key in ef:
        assert torch.isfinite(gf[key]).all() and torch.isfinite(gr[key]).all(), key
        assert torch.equal(gf[key], ef[key]), f"forward scan {key}"
        assert torch.equal(gr[key], er[key]), f"reverse scan {key}"


def test_backward_bidir_against_the_oracle():
    """Both scans' gradients of one bidirectional call at the 720p width, 700 tokens, 2 heads."""
    B, T, H, D = 1, 700, 2, 112
    d = gdn_inputs.batch(82, B, T, H, D, with_state=True)
    dO, dSf, _ = _bidir_inputs(d, D, T, 82)
    ref_f = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO[0].float().numpy(), d["S0"], dSf.numpy())
    ref_r = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO[1].float().numpy(), None, None, reverse=True)
    s = gb.Stream(B, H, D, D, T, poison_ws=True)
    try:
        t = dev_inputs(d)
        S0 = torch.from_numpy(np.ascontiguousarray(d["S0"], np.float32)).cuda()
        gf, gr = s.backward_bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], dO[0].cuda(), dO[1].cuda(),
                                  d_state=dSf.cuda(), state0=S0)
        torch.cuda.synchronize()
    finally:
        s.close()
    print("forward scan:", flush=True)
    _check_all(gf, ref_f)
    print("reverse scan:", flush=True)
    _check_all(gr, ref_r)


def test_backward_bidir_rejects_a_start_state_for_the_reverse_scan():
    """g_rev->state0 set, or g_rev missing: GDN_E_INVAL and nothing written."""
    B, T, H, D = 1, 40, 2, 32
    d = gdn_inputs.batch(83, B, T, H, D, with_state=True)
    dO, dSf, _ = _bidir_inputs(d, D, T, 83)
    s = gb.Stream(B, H, D, D, T, poison_ws=True)
    try:
        t = dev_inputs(d)
        S0 = torch.from_numpy(np.ascontiguousarray(d["S0"], np.float32)).cuda()
        args = (t["q"], t["k"], t["v"], t["a"], t["beta"])
        gf, gr = s._grad_buffers(t["q"], t["v"]), s._grad_buffers(t["q"], t["v"])
        for x in list(gf.values()) + list(gr.values()):
            x.fill_(7.0)
        io = gb._make_io(t["q"], t["k"], t["v"], dO[0].cuda(), t["a"], t["beta"])
        g_f = gb._make_grad(dO[0].cuda(), gf, dSf.cuda(), S0)
        g_r = gb._make_grad(dO[1].cuda(), gr, None, S0)
        lib = gb.load_library()
        import ctypes
        rc = lib.gdn_chunk_backward_bidir(ctypes.c_void_p(s.handle), ctypes.byref(io), ctypes.byref(g_f),
                                          ctypes.byref(g_r), T, None)
        assert rc == gb.GDN_E_INVAL and "state0" in gb.gdn_last_error()
        rc = lib.gdn_chunk_backward_bidir(ctypes.c_void_p(s.handle), ctypes.byref(io), ctypes.byref(g_f), None, T, None)
        assert rc == gb.GDN_E_INVAL and "g_rev" in gb.gdn_last_error()
        torch.cuda.synchronize()
        for x in list(gf.values()) + list(gr.values()):
            assert bool((x == 7.0).all())
    finally:
        s.close()


@pytest.mark.parametrize("T", [1, 7, 8, 9, 17, 63, 65, 129])
def test_backward_staging_block_edges(T):
    """Lengths around the 8-token staging block (one token, a short block, exactly one block, one
    token into the second, two blocks and one) and the 64-token walk segment (one short of a segment,
    one token into the second, two segments and one), both scans through the bidirectional call,
    against the oracle."""
    B, H, D = 1, 2, 32
    d = gdn_inputs.batch(90 + T, B, T, H, D, with_state=True)
    dO, dSf, dSr = _bidir_inputs(d, D, T, 90 + T)
    ref_f = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO[0].float().numpy(), d["S0"], dSf.numpy())
    ref_r = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO[1].float().numpy(), None, dSr.numpy(),
                            reverse=True)
    s = gb.Stream(B, H, D, D, T, poison_ws=True)
    try:
        t = dev_inputs(d)
        S0 = torch.from_numpy(np.ascontiguousarray(d["S0"], np.float32)).cuda()
        gf, gr = s.backward_bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], dO[0].cuda(), dO[1].cuda(),
                                  d_state=dSf.cuda(), state0=S0, d_state_rev=dSr.cuda())
        torch.cuda.synchronize()
    finally:
        s.close()
    _check_all(gf, ref_f)
    _check_all(gr, ref_r)
