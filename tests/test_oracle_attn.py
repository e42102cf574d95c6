"""Pins of the sliding-window + persistent-sink attention oracle (oracle/window_attn.py).

The oracle is checked against what does not depend on its own code: torch's fp64
scaled_dot_product_attention on the CPU (a library routine), closed forms (zero query, one
dominant key, a hand-computed two-key example), the hand-derived visibility table in
tests/golden/attn_visibility.txt read back through the outputs, and equivalences that follow
from the cache reading (a cache that holds everything is block-causal attention over the whole
stream; a window of one chunk is attention over two chunks).  A planted mistake in a copy of the
oracle must fail at least one of them.
"""
import os
import types

import numpy as np
import pytest
import torch

from oracle import window_attn as wa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attn_visibility.txt")
ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "window_attn.py")


def _sdpa(q, k, v, scale, mask=None):
    """torch's fp64 CPU attention for one head: q [n, d], k [m, d], v [m, dv]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return o[0, 0].numpy()


def _load_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "case":
            cur = {"name": f[1], "n_sink": int(f[2]), "n_window": int(f[3]), "calls": []}
            cases.append(cur)
        else:
            cur["calls"].append((int(f[1]), bool(int(f[2])), [int(x) for x in f[3:]]))
    return cases


# ---- the pin battery (also run against planted mistakes) -------------------------------------

def _pin_sdpa(m):
    rng = np.random.default_rng(3)
    for n, mk, d, dv, scale in [(5, 7, 4, 3, 0.7), (9, 33, 16, 16, None), (1, 1, 3, 2, 2.0)]:
        q, k, v = rng.normal(size=(n, d)), rng.normal(size=(mk, d)), rng.normal(size=(mk, dv))
        s = scale if scale is not None else 1 / np.sqrt(d)
        if not np.allclose(m.attend(q, k, v, s), _sdpa(q, k, v, s), rtol=1e-12, atol=1e-13):
            return False
    return True


def _pin_closed_forms(m):
    rng = np.random.default_rng(4)
    k, v = rng.normal(size=(6, 5)), rng.normal(size=(6, 3))
    # zero query: uniform weights, the mean of the values
    if not np.allclose(m.attend(np.zeros((2, 5)), k, v, 0.9), np.tile(v.mean(0), (2, 1)), rtol=0, atol=1e-14):
        return False
    # one key 60 logits above the rest: its value (the others weigh e^-60 ~ 1e-26)
    q = np.zeros((1, 5)); q[0, 0] = 1.0
    kk = np.zeros((6, 5)); kk[2, 0] = 60.0
    if not np.allclose(m.attend(q, kk, v, 1.0), v[2:3], rtol=0, atol=1e-20):
        return False
    # two keys with logits 0 and ln 3: weights 1/4 and 3/4, values (4, 0) and (0, 8) -> (1, 6)
    o = m.attend(np.array([[1.0, 0.0]]), np.array([[0.0, 0.0], [np.log(3.0), 0.0]]),
                 np.array([[4.0, 0.0], [0.0, 8.0]]), 1.0)
    return np.allclose(o, [[1.0, 6.0]], rtol=0, atol=1e-14)


def _pin_visibility(m):
    """Zero queries and one-hot values: the output of each query is 1/n on every token it sees."""
    for case in _load_cases():
        total = sum(T for T, _, _ in case["calls"])
        att = m.SinkWindowAttention(case["n_sink"], case["n_window"], scale=1.0)
        hist_ids, next_id = [], 0
        for T, commit, vis in case["calls"]:
            ids = list(range(next_id, next_id + T))
            next_id += T
            eye = np.eye(total)[ids]                             # [T, total]
            q = np.zeros((1, T, 1, 2))
            k = np.random.default_rng(next_id).normal(size=(1, T, 1, 2))
            o = att.chunk(q, k, eye[None, :, None, :], commit=commit)
            want = np.zeros(total)
            seen = [hist_ids[i] for i in vis] + ids
            want[seen] = 1.0 / len(seen)
            if not np.allclose(o[0, :, 0], np.tile(want, (T, 1)), rtol=0, atol=1e-15):
                return False
            if commit:
                hist_ids += ids
    return True


def _pin_block_causal(m):
    """A cache that holds everything: chunk c sees all tokens up to the end of chunk c."""
    rng = np.random.default_rng(5)
    B, H, d, sizes = 2, 2, 8, [3, 5, 4]
    N = sum(sizes)
    q, k, v = (rng.normal(size=(B, N, H, d)) for _ in range(3))
    att = m.SinkWindowAttention(2, N, scale=None)
    outs, t0 = [], 0
    for T in sizes:
        outs.append(att.chunk(q[:, t0:t0 + T], k[:, t0:t0 + T], v[:, t0:t0 + T]))
        t0 += T
    o = np.concatenate(outs, axis=1)
    ends = np.cumsum(sizes)
    last = np.repeat(ends, sizes)                              # end of each query's chunk
    mask = np.arange(N)[None, :] < last[:, None]
    for b in range(B):
        for h in range(H):
            ref = _sdpa(q[b, :, h], k[b, :, h], v[b, :, h], 1 / np.sqrt(d), mask)
            if not np.allclose(o[b, :, h], ref, rtol=1e-12, atol=1e-13):
                return False
    return True


def _pin_two_chunks(m):
    """No sink, a window of one chunk: chunk c sees exactly chunks c-1 and c."""
    rng = np.random.default_rng(6)
    T, d, n = 4, 6, 4
    q, k, v = (rng.normal(size=(1, n * T, 1, d)) for _ in range(3))
    att = m.SinkWindowAttention(0, T, scale=0.5)
    for c in range(n):
        s = slice(c * T, (c + 1) * T)
        o = att.chunk(q[:, s], k[:, s], v[:, s])
        lo = max(0, c - 1) * T
        ref = _sdpa(q[0, s, 0], k[0, lo:(c + 1) * T, 0], v[0, lo:(c + 1) * T, 0], 0.5)
        if not np.allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-13):
            return False
    return True


def _pin_no_commit(m):
    rng = np.random.default_rng(7)
    q, k, v = (rng.normal(size=(1, 3, 2, 4)) for _ in range(3))
    att = m.SinkWindowAttention(1, 2)
    att.chunk(q, k, v)
    a = att.chunk(q * 2, k, v, commit=False)
    b = att.chunk(q * 2, k, v, commit=False)
    return att.history == 3 and np.array_equal(a, b)


PINS = [_pin_sdpa, _pin_closed_forms, _pin_visibility, _pin_block_causal, _pin_two_chunks, _pin_no_commit]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__[5:])
def test_oracle_pin(pin):
    assert pin(wa)


def test_golden_cases_parse():
    cases = _load_cases()
    assert [c["name"] for c in cases] == ["A", "B", "C"]
    assert sum(len(c["calls"]) for c in cases) == 14


# ---- planted mistakes -------------------------------------------------------------------------

MUTANTS = {
    "window_one_short": ("start = max(n_sink, history - n_window)", "start = max(n_sink, history - n_window + 1)"),
    "sink_repeated_in_window": ("start = max(n_sink, history - n_window)", "start = max(0, history - n_window)"),
    "window_from_oldest": ("return sink + list(range(start, history))",
                           "return sink + list(range(n_sink, min(history, n_sink + n_window)))"),
    "sink_dropped": ("sink = list(range(min(history, n_sink)))", "sink = []"),
    "own_chunk_unseen": ("keys = np.concatenate([self.k_hist[b, idx, h], k[b, :, h]])",
                         "keys = np.concatenate([self.k_hist[b, idx, h], 0 * k[b, :, h]])"),
    "scale_ignored": ("logits = scale * (q @ k.T)", "logits = q @ k.T"),
    "normalised_over_queries": ("w.sum(axis=1, keepdims=True)", "w.sum(axis=0, keepdims=True)"),
    "no_commit_commits": ("if commit:", "if True:"),
    "default_scale_inverted": ("1.0 / np.sqrt(d)", "np.sqrt(d)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"anchor of {name} not unique"
    mod = types.ModuleType("window_attn_" + name)
    exec(compile(src.replace(old, new), ORACLE_SRC + ":" + name, "exec"), mod.__dict__)
    def passes(pin):
        try:
            return pin(mod)
        except Exception:      # a mistake that breaks the computation outright is caught too
            return False
    assert not all(passes(p) for p in PINS), f"no pin catches {name}"
