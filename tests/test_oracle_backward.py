"""Pins of the oracle's gradient (``oracle.backward``) against central finite differences of
the oracle's own scan in fp64.  Every input of the scan is perturbed entry by entry, so a
dropped term, a wrong sign or a transposed operand anywhere in the backward fails here.

The loss is L = <dO, o> + <dS_final, S_T> with random weights, so its gradients with respect
to o and S_T are dO and dS_final."""
import numpy as np
import pytest

import oracle


def _case(seed, B=1, T=7, H=2, Dk=4, Dv=3, start=True):
    rng = np.random.default_rng(seed)
    d = {
        "q": rng.standard_normal((B, T, H, Dk)),
        "k": rng.standard_normal((B, T, H, Dk)),
        "v": rng.standard_normal((B, T, H, Dv)),
        "a": rng.uniform(0.5, 1.0, (B, T, H)),
        "beta": rng.uniform(0.05, 1.0, (B, T, H)),
        "S0": 0.3 * rng.standard_normal((B, H, Dv, Dk)) if start else None,
    }
    dO = rng.standard_normal((B, T, H, Dv))
    dSf = rng.standard_normal((B, H, Dv, Dk))
    return d, dO, dSf


def _loss(d, dO, dSf, **kw):
    o, S = oracle.scan(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], threads=1, **kw)
    return float((o * dO).sum() + (S * dSf).sum())


def _fd(d, name, dO, dSf, h=1e-6, **kw):
    x = d[name]
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        keep = x[i]
        x[i] = keep + h
        lp = _loss(d, dO, dSf, **kw)
        x[i] = keep - h
        lm = _loss(d, dO, dSf, **kw)
        x[i] = keep
        g[i] = (lp - lm) / (2 * h)
    return g


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("l2norm", [True, False])
def test_backward_matches_finite_differences(reverse, l2norm):
    d, dO, dSf = _case(11 + 2 * reverse + l2norm)
    kw = dict(reverse=reverse, l2norm=l2norm, scale=0.7)
    if not l2norm:
        # keep I - beta k k^T contractive without the normalisation
        d["k"] *= 0.4
    g = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO, d["S0"], dSf, threads=1, **kw)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "da"), ("beta", "dbeta"), ("S0", "dS0")):
        fd = _fd(d, name, dO, dSf, **kw)
        err = np.abs(g[key] - fd).max()
        assert err <= 1e-6 * max(1.0, np.abs(fd).max()), (name, err)


def test_backward_zero_start_and_no_final_gradient():
    """Without a start state the gradient of the (zero) start state is still returned; without
    dS_final only the output term drives the gradients."""
    d, dO, _ = _case(23, start=False)
    g = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO, None, None, threads=1)
    d["S0"] = np.zeros((1, 2, 3, 4))
    zero = np.zeros((1, 2, 3, 4))
    for name, key in (("k", "dk"), ("beta", "dbeta"), ("S0", "dS0")):
        fd = _fd(d, name, dO, zero)
        assert np.abs(g[key] - fd).max() <= 1e-6 * max(1.0, np.abs(fd).max()), name


def test_backward_of_identity_rule():
    """a = 1, beta = 0: S_t = S0 for all t, o_t = S0 q_t.  Then dv = 0, dS0 = dS_final +
    scale sum_t do_t q_t^T and dq_t = scale S0^T do_t (normalisation off)."""
    d, dO, dSf = _case(31)
    d["a"][:] = 1.0
    d["beta"][:] = 0.0
    g = oracle.backward(d["q"], d["k"], d["v"], d["a"], d["beta"], dO, d["S0"], dSf, l2norm=False,
                        scale=0.5, threads=1)
    assert np.abs(g["dv"]).max() == 0.0
    want_S0 = dSf + 0.5 * np.einsum("bthv,bthk->bhvk", dO, d["q"])
    assert np.allclose(g["dS0"], want_S0, rtol=1e-12, atol=1e-12)
    want_dq = 0.5 * np.einsum("bhvk,bthv->bthk", d["S0"], dO)
    assert np.allclose(g["dq"], want_dq, rtol=1e-12, atol=1e-12)
