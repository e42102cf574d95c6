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
    s = gb.Stream(B, H, D, Dv, max(T, 1), io_dtype=io)
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
@pytest.mark.parametrize("D", [16, 32, 112])
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


@pytest.mark.parametrize("reverse", [False, True])
def test_backward_720p_width_long(reverse):
    """d = 112, 700 tokens (several hundred steps of gradient flow through the state)."""
    d = gdn_inputs.batch(77, 1, 700, 2, 112, with_state=True)
    g, ref = _grads(d, 112, 112, 700, reverse=reverse, seed=77)
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
