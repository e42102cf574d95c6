"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-derived worked
examples (tests/golden), an independent closed form (explicit products of the
per-token transition matrices), special cases with known answers, invariants
named for the method (chunked = token-sequential, carried state = one long
scan, reverse = forward on time-reversed input, a=1/beta=0 keeps the state,
beta=1 with a unit key erases the state along that key) and the contraction
bound of the delta rule.
"""
import glob
import os

import numpy as np
import pytest

import gdn_inputs
from oracle.chunked import chunked_scan

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, B, T, H, Dk, Dv, state=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    a = np.exp(-0.1 * np.logaddexp(0, rng.standard_normal((B, T, H))))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, Dv, Dk)) if state else None
    return q, k, v, a, beta, S0


def _closed_form_head(q, k, v, a, beta, S0, *, reverse, l2norm, eps, scale):
    """Unrolled form: with A_t = a_t (I - beta_t k^_t k^_t^T) and the scan order p_1..p_n,
    S after token p_n = S0 A_{p_1}...A_{p_n} + sum_j beta_{p_j} v_{p_j} k^_{p_j}^T A_{p_{j+1}}...A_{p_n}."""
    T, Dk = q.shape
    nrm = (lambda x: x / np.sqrt(np.sum(x * x) + eps)) if l2norm else (lambda x: x)
    kh = [nrm(k[t]) for t in range(T)]
    qh = [nrm(q[t]) for t in range(T)]
    A = [a[t] * (np.eye(Dk) - beta[t] * np.outer(kh[t], kh[t])) for t in range(T)]
    order = list(range(T))[::-1] if reverse else list(range(T))
    o = np.zeros((T, v.shape[1]))
    S = S0.copy()
    for n in range(1, T + 1):
        seq = order[:n]

        def chain(idx):
            P = np.eye(Dk)
            for m in idx:
                P = P @ A[m]
            return P

        S = S0 @ chain(seq)
        for j, t in enumerate(seq):
            S = S + beta[t] * np.outer(v[t], kh[t]) @ chain(seq[j + 1:])
        o[seq[-1]] = scale * S @ qh[seq[-1]]
    return o, S


def _load_golden(path):
    d = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = [float(x) for x in vals]
    Dk, Dv, T = int(d["Dk"][0]), int(d["Dv"][0]), int(d["T"][0])
    return dict(
        q=np.array(d["q"]).reshape(1, T, 1, Dk), k=np.array(d["k"]).reshape(1, T, 1, Dk),
        v=np.array(d["v"]).reshape(1, T, 1, Dv), a=np.array(d["a"]).reshape(1, T, 1),
        beta=np.array(d["beta"]).reshape(1, T, 1), S0=np.array(d["S0"]).reshape(1, 1, Dv, Dk),
        o=np.array(d["o"]).reshape(1, T, 1, Dv), S=np.array(d["S"]).reshape(1, 1, Dv, Dk),
        l2norm=bool(d["l2norm"][0]), eps=d["eps"][0], scale=d["scale"][0],
        reverse=bool(d["reverse"][0]))


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "hand_*.txt"))),
                         ids=lambda p: os.path.basename(p))
def test_golden_hand_examples(oracle_lib, path):
    g = _load_golden(path)
    o, S = oracle_lib.scan(g["q"], g["k"], g["v"], g["a"], g["beta"], g["S0"], reverse=g["reverse"],
                           l2norm=g["l2norm"], eps=g["eps"], scale=g["scale"], threads=1)
    np.testing.assert_allclose(o, g["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(S, g["S"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("reverse", [False, True])
@pytest.mark.parametrize("l2norm", [True, False])
@pytest.mark.parametrize("dims", [(5, 3, 9), (8, 8, 12), (3, 6, 7)])
def test_brute_force_closed_form(oracle_lib, reverse, l2norm, dims):
    Dk, Dv, T = dims
    rng = np.random.default_rng(100 + Dk * 7 + Dv * 3 + T)
    q, k, v, a, beta, S0 = _rand_case(rng, 2, T, 2, Dk, Dv)
    if not l2norm:                     # keep the transitions contractive without normalisation
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o, S = oracle_lib.scan(q, k, v, a, beta, S0, reverse=reverse, l2norm=l2norm, eps=1e-6,
                           scale=0.75, threads=3, row_block=2)
    for b in range(2):
        for h in range(2):
            oe, Se = _closed_form_head(q[b, :, h], k[b, :, h], v[b, :, h], a[b, :, h], beta[b, :, h],
                                       S0[b, h], reverse=reverse, l2norm=l2norm, eps=1e-6, scale=0.75)
            np.testing.assert_allclose(o[b, :, h], oe, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(S[b, h], Se, rtol=1e-12, atol=1e-13)


def test_identity_when_a1_beta0(oracle_lib):
    """a = 1, beta = 0: the state never changes and o_t = S0 q^_t."""
    rng = np.random.default_rng(1)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 40, 3, 16, 16)
    a[:] = 1.0
    beta[:] = 0.0
    o, S = oracle_lib.scan(q, k, v, a, beta, S0)
    assert np.array_equal(S, S0)
    qh = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(o, np.einsum("bhrc,bthc->bthr", S0, qh), rtol=1e-13, atol=1e-14)


def test_pure_decay_when_beta0(oracle_lib):
    """beta = 0: S_t = (prod_{s<=t} a_s) S0."""
    rng = np.random.default_rng(2)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 30, 2, 8, 8)
    beta[:] = 0.0
    _, S = oracle_lib.scan(q, k, v, a, beta, S0)
    np.testing.assert_allclose(S, np.prod(a, axis=1)[:, :, None, None] * S0, rtol=1e-13)


def test_orthonormal_keys_write_columns(oracle_lib):
    """a = 1, beta = 1, S0 = 0, k_t = e_t: S_T = sum_t v_t e_t^T (column t of S is v_t)."""
    D, T = 12, 9
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, T, 1, D))
    k = np.zeros((1, T, 1, D))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    v = rng.standard_normal((1, T, 1, D))
    ones = np.ones((1, T, 1))
    _, S = oracle_lib.scan(q, k, v, ones, ones, None, l2norm=False)
    expect = np.zeros((D, D))
    expect[:, :T] = v[0, :, 0].T
    np.testing.assert_allclose(S[0, 0], expect, rtol=0, atol=1e-15)


def test_erase_along_unit_key(oracle_lib):
    """a = 1, beta = 1, v = 0, unit k: S_t k = 0 and S_t x = S_{t-1} x for x orthogonal to k."""
    rng = np.random.default_rng(4)
    D = 10
    S0 = rng.standard_normal((1, 1, D, D))
    k = rng.standard_normal(D)
    k /= np.linalg.norm(k)
    kk = k.reshape(1, 1, 1, D)
    z = np.zeros((1, 1, 1, D))
    ones = np.ones((1, 1, 1))
    _, S = oracle_lib.scan(z, kk, z, ones, ones, S0, l2norm=False)
    np.testing.assert_allclose(S[0, 0] @ k, 0.0, atol=1e-14)
    x = rng.standard_normal(D)
    x -= (x @ k) * k
    np.testing.assert_allclose(S[0, 0] @ x, S0[0, 0] @ x, rtol=1e-13, atol=1e-14)


def test_linearity_in_state_and_values(oracle_lib):
    """o and S are linear in (S0, v) jointly: superposition and scaling."""
    rng = np.random.default_rng(5)
    q, k, v1, a, beta, S1 = _rand_case(rng, 1, 25, 2, 8, 8)
    _, _, v2, _, _, S2 = _rand_case(rng, 1, 25, 2, 8, 8)
    o1, F1 = oracle_lib.scan(q, k, v1, a, beta, S1)
    o2, F2 = oracle_lib.scan(q, k, v2, a, beta, S2)
    o3, F3 = oracle_lib.scan(q, k, 2 * v1 - 3 * v2, a, beta, 2 * S1 - 3 * S2)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(F3, 2 * F1 - 3 * F2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C", [16, 64, 80])
@pytest.mark.parametrize("reverse", [False, True])
def test_chunked_equals_token_sequential(oracle_lib, C, reverse):
    """Invariant 1: the chunkwise rewrite (with a ragged last chunk) equals the per-token rule."""
    rng = np.random.default_rng(6 + C)
    q, k, v, a, beta, S0 = _rand_case(rng, 2, 203, 2, 16, 16)
    S0 = None if reverse else S0
    o, S = oracle_lib.scan(q, k, v, a, beta, S0, reverse=reverse)
    oc, Sc = chunked_scan(q, k, v, a, beta, S0, C=C, reverse=reverse)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


def test_chunked_equals_token_sequential_head_dim_112(oracle_lib):
    rng = np.random.default_rng(7)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 150, 1, 112, 112)
    o, S = oracle_lib.scan(q, k, v, a, beta, S0)
    oc, Sc = chunked_scan(q, k, v, a, beta, S0, C=64)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-12)


def test_carried_state_equals_one_long_scan(oracle_lib):
    """Invariant 4: chunk-by-chunk with the carried state is bitwise one long scan."""
    d = gdn_inputs.batch(9, 2, 8 * 50, 2, 16, with_state=True)
    o_long, S_long = oracle_lib.scan(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"])
    S = d["S0"]
    for c in range(8):
        sl = slice(50 * c, 50 * (c + 1))
        o_c, S = oracle_lib.scan(d["q"][:, sl], d["k"][:, sl], d["v"][:, sl], d["a"][:, sl],
                                 d["beta"][:, sl], S)
        assert np.array_equal(o_c, o_long[:, sl])
    assert np.array_equal(S, S_long)


def test_reverse_is_forward_on_flipped_input(oracle_lib):
    """Invariant 5: reverse(x) = flip(forward(flip(x))), bitwise."""
    d = gdn_inputs.batch(9, 2, 77, 3, 16)
    f = lambda x: np.ascontiguousarray(x[:, ::-1])
    o_r, S_r = oracle_lib.scan(d["q"], d["k"], d["v"], d["a"], d["beta"], None, reverse=True)
    o_f, S_f = oracle_lib.scan(f(d["q"]), f(d["k"]), f(d["v"]), f(d["a"]), f(d["beta"]), None)
    assert np.array_equal(o_r, f(o_f))
    assert np.array_equal(S_r, S_f)


def test_partition_does_not_change_result(oracle_lib):
    """Rows of S evolve independently: thread count and row blocking are bitwise irrelevant."""
    d = gdn_inputs.batch(9, 2, 60, 3, 20, with_state=True)
    args = (d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"])
    o1, S1 = oracle_lib.scan(*args, threads=1, row_block=20)
    o2, S2 = oracle_lib.scan(*args, threads=5, row_block=3)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_contraction_bound(oracle_lib):
    """With unit keys and beta in [0, 2], ||I - beta k k^T||_2 <= 1, so
    ||S_t||_F <= a_t ||S_{t-1}||_F + beta_t ||v_t||; chained over every prefix."""
    rng = np.random.default_rng(8)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 24, 1, 8, 8)
    beta = 2.0 * rng.random((1, 24, 1))
    bound = np.linalg.norm(S0[0, 0])
    for t in range(24):
        _, S = oracle_lib.scan(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], a[:, :t + 1],
                               beta[:, :t + 1], S0)
        bound = a[0, t, 0] * bound + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S[0, 0]) <= bound * (1 + 1e-12)


def test_empty_sequence_returns_start_state(oracle_lib):
    rng = np.random.default_rng(10)
    q, k, v, a, beta, S0 = _rand_case(rng, 1, 0, 2, 4, 4)
    o, S = oracle_lib.scan(q, k, v, a, beta, S0)
    assert o.shape == (1, 0, 2, 4) and np.array_equal(S, S0)
