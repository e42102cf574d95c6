"""GPU parity on the streaming workloads: carried state over consecutive chunks,
many layers with replay of the same cached states, a long stream checked for
drift, a long bidirectional clip, and the state-cache semantics (checkpoint and
resume, no-commit replay, repeatability).

Every comparison is against the fp64 oracle run on the same seeded inputs, at
the tolerance of this path (max-abs 2e-2, relative Frobenius 5e-3) for every
chunk, direction and state.  Every handle fills its workspace with NaN bytes at init
(GDN_POISON_WS), so a read of a workspace byte the kernels did not write shows up.
"""
import numpy as np
import pytest

import gdn_inputs
import oracle
from tests.gpu_util import assert_close, dev_inputs, metrics, TOL_MAX_ABS, TOL_REL_F

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402

T1, H1, D1 = gdn_inputs.CHUNK_TOKENS, gdn_inputs.HEADS, gdn_inputs.HEAD_DIM


def _fwd_rev(s, t, **kw):
    o_f, o_r = torch.empty_like(t["v"]), torch.empty_like(t["v"])
    s.bidir(t["q"], t["k"], t["v"], t["a"], t["beta"], o_f, o_r, **kw)
    return o_f, o_r


def test_streaming_8_chunks_4_streams():
    """The 720p layer over 8 consecutive 2640-token chunks, B=4 independent streams, the
    state cache carried chunk to chunk; each chunk runs the forward and the reverse scan."""
    B, n_chunks = 4, 8
    s = gb.Stream(B, H1, D1, D1, T1, poison_ws=True)
    try:
        d0 = gdn_inputs.batch(2, B, T1, H1, D1, chunk=0, with_state=True)
        S_ref = d0["S0"].astype(np.float64)
        s.state_set(torch.from_numpy(d0["S0"]).cuda())
        for c in range(n_chunks):
            d = d0 if c == 0 else gdn_inputs.batch(2, B, T1, H1, D1, chunk=c)
            t = dev_inputs(d)
            o_f, o_r = _fwd_rev(s, t)
            S = s.state_get()
            torch.cuda.synchronize()
            of, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S_ref)
            orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"])
            print(f"chunk {c}", flush=True)
            assert_close("o_fwd", o_f, of)
            assert_close("o_rev", o_r, orv)
            assert_close("state", S, S_ref)
    finally:
        s.close()


def _c3_layers(step):
    return [gdn_inputs.batch(3, 1, T1, H1, D1, layer=l, step=step, with_state=(step == 0))
            for l in range(gdn_inputs.GDN_LAYERS)]


def _stack(ds):
    return {k: np.concatenate([d[k] for d in ds]) for k in ds[0]}


def test_15_layers_two_denoising_steps_batched():
    """15 independent GDN layers as one B=15 handle, 2 denoising steps replaying the same
    cached states: step 1 with GDN_NO_COMMIT (the cache must stay bitwise unchanged and the
    final state goes to state_out), step 2 on fresh inputs, committed."""
    L = gdn_inputs.GDN_LAYERS
    s = gb.Stream(L, H1, D1, D1, T1, poison_ws=True)
    try:
        step0 = _stack(_c3_layers(0))
        S0 = step0["S0"]
        s.state_set(torch.from_numpy(S0).cuda())
        cache_before = s.state_get().cpu().numpy().copy()
        for step in range(2):
            d = step0 if step == 0 else _stack(_c3_layers(1))
            t = dev_inputs(d)
            if step == 0:
                S_out = torch.empty((L, H1, D1, D1), dtype=torch.float32, device="cuda")
                o_f, o_r = _fwd_rev(s, t, flags=gb.GDN_NO_COMMIT, state_out=S_out)
            else:
                o_f, o_r = _fwd_rev(s, t)
                S_out = s.state_get()
            torch.cuda.synchronize()
            of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S0)
            orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"])
            print(f"denoising step {step}", flush=True)
            assert_close("o_fwd", o_f, of)
            assert_close("o_rev", o_r, orv)
            assert_close("state", S_out, Sf)
            if step == 0:
                cache = s.state_get().cpu().numpy()
                assert np.array_equal(cache.view(np.uint32), cache_before.view(np.uint32)), \
                    "GDN_NO_COMMIT changed the cache"
    finally:
        s.close()


def test_15_layers_independent_handles():
    """The same 15-layer step with one handle per layer (batch 1 each) matches the batched
    handle bitwise, and the oracle."""
    L = gdn_inputs.GDN_LAYERS
    layers = _c3_layers(0)
    d = _stack(layers)
    sb = gb.Stream(L, H1, D1, D1, T1, poison_ws=True)
    try:
        sb.state_set(torch.from_numpy(d["S0"]).cuda())
        ob_f, ob_r = _fwd_rev(sb, dev_inputs(d))
        Sb = sb.state_get()
        torch.cuda.synchronize()
    finally:
        sb.close()
    of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"])
    for l, dl in enumerate(layers):
        s = gb.Stream(1, H1, D1, D1, T1, poison_ws=True)
        try:
            s.state_set(torch.from_numpy(dl["S0"]).cuda())
            o_f, o_r = _fwd_rev(s, dev_inputs(dl))
            S = s.state_get()
            torch.cuda.synchronize()
        finally:
            s.close()
        assert torch.equal(o_f, ob_f[l:l + 1]) and torch.equal(o_r, ob_r[l:l + 1])
        assert torch.equal(S, Sb[l:l + 1])
        if l in (0, L - 1):
            assert_close(f"layer {l} o_fwd", o_f, of[l:l + 1])
            assert_close(f"layer {l} state", S, Sf[l:l + 1])


@pytest.mark.timeout(900)
def test_200_chunk_stream_drift(tmp_path):
    """The 720p layer over 200 consecutive chunks (600 latent frames, 528k tokens) with the
    carried state: every chunk's o, o_rev and state, all 20 heads, must meet the tolerance
    against one long fp64 oracle scan.  Inputs follow the seeded scheme of every other case
    (SeedSequence([4, 0, 0, chunk, 0]) -> PCG64, gdn_inputs.batch), drawn ahead in a small pool
    of worker processes.  The per-chunk error series and its fitted slope are written to
    drift_c4a.json (in $GDN_RESULTS_DIR when set, else the test's temporary folder) and the
    assertions read them back from there: every chunk within tolerance, and a fitted growth
    of the state error over the 200 chunks below a fifth of the tolerance (with gates that
    forget within about a hundred tokens the error must not accumulate)."""
    import concurrent.futures as cf
    import json
    import multiprocessing as mp
    import os

    n_chunks, ahead = 200, 8
    threads = min(16, oracle.default_threads())
    s = gb.Stream(1, H1, D1, D1, T1, poison_ws=True)
    series = []
    with cf.ProcessPoolExecutor(max_workers=6, mp_context=mp.get_context("spawn")) as pool:
        def submit(c):
            return pool.submit(gdn_inputs.batch, 4, 1, T1, H1, D1, chunk=c, with_state=(c == 0))
        pending = {c: submit(c) for c in range(min(ahead, n_chunks))}
        try:
            S_ref = None
            for c in range(n_chunks):
                d = pending.pop(c).result()
                if c + ahead < n_chunks:
                    pending[c + ahead] = submit(c + ahead)
                t = dev_inputs(d)
                if c == 0:
                    s.state_set(torch.from_numpy(d["S0"]).cuda())
                    S_ref = d["S0"].astype(np.float64)
                o_f, o_r = _fwd_rev(s, t)
                S = s.state_get()
                of, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S_ref, threads=threads)
                orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"], threads=threads)
                torch.cuda.synchronize()
                e = [metrics(o_f, of), metrics(o_r, orv), metrics(S, S_ref)]
                series.append([x for pair in e for x in pair])
                if c % 20 == 0:
                    print(f"chunk {c}: rel_F o_fwd {e[0][1]:.3e} o_rev {e[1][1]:.3e} state {e[2][1]:.3e}", flush=True)
        finally:
            s.close()
    errs = np.array(series)
    slopes = {name: float(np.polyfit(np.arange(n_chunks), errs[:, i], 1)[0])
              for i, name in enumerate(("o_fwd_max_abs", "o_fwd_rel_F", "o_rev_max_abs", "o_rev_rel_F",
                                        "state_max_abs", "state_rel_F"))}
    out_dir = os.environ.get("GDN_RESULTS_DIR") or str(tmp_path)
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, "drift_c4a.json")
    with open(path, "w") as f:
        json.dump({"workload": "B=1 H=20 d=112, 200 chunks x 2640 tokens, carried state, fwd + rev",
                   "columns": ["o_fwd_max_abs", "o_fwd_rel_F", "o_rev_max_abs", "o_rev_rel_F", "state_max_abs",
                               "state_rel_F"],
                   "per_chunk": errs.tolist(), "slope_per_chunk": slopes,
                   "tolerance": {"max_abs": TOL_MAX_ABS, "rel_F": TOL_REL_F}}, f)
    print(f"drift series written to {path}", flush=True)
    with open(path) as f:
        rec = json.load(f)
    e = np.array(rec["per_chunk"])
    assert e.shape == (n_chunks, 6)
    for c, row in enumerate(e):
        for i, name in enumerate(("o_fwd", "o_rev", "state")):
            assert row[2 * i] <= TOL_MAX_ABS and row[2 * i + 1] <= TOL_REL_F, \
                f"chunk {c} {name}: max_abs {row[2 * i]:.3e} rel_F {row[2 * i + 1]:.3e}"
    growth = rec["slope_per_chunk"]["state_rel_F"] * n_chunks
    print(f"drift over {n_chunks} chunks: max rel_F o_fwd {e[:, 1].max():.3e}, o_rev {e[:, 3].max():.3e}, "
          f"state {e[:, 5].max():.3e}; state rel_F slope {rec['slope_per_chunk']['state_rel_F']:.2e} per chunk "
          f"({growth:.2e} over the stream)", flush=True)
    assert growth <= 0.2 * TOL_REL_F


def test_long_bidirectional_clip():
    """A full bidirectional scan over 21 latent frames x 880 tokens = 18480 tokens, H=20, d=112:
    forward and reverse, both from a zero state."""
    T = 21 * gdn_inputs.TOKENS_PER_FRAME
    d = gdn_inputs.batch(5, 1, T, H1, D1)
    s = gb.Stream(1, H1, D1, D1, T, poison_ws=True)
    try:
        t = dev_inputs(d)
        o_f, o_r = _fwd_rev(s, t)
        S = s.state_get()
        torch.cuda.synchronize()
    finally:
        s.close()
    of, Sf = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"])
    orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"])
    assert_close("o_fwd", o_f, of)
    assert_close("o_rev", o_r, orv)
    assert_close("state", S, Sf)


def test_checkpoint_and_resume_is_bitwise():
    """Saving the cache after chunk 1 (gdn_state_get) and restoring it into a fresh handle
    (gdn_state_set) continues the stream bitwise as if it had not been interrupted."""
    d1 = gdn_inputs.batch(6, 2, T1, 4, D1, chunk=0, with_state=True)
    d2 = gdn_inputs.batch(6, 2, T1, 4, D1, chunk=1)
    a = gb.Stream(2, 4, D1, D1, T1, poison_ws=True)
    b = gb.Stream(2, 4, D1, D1, T1, poison_ws=True)
    try:
        a.state_set(torch.from_numpy(d1["S0"]).cuda())
        t1, t2 = dev_inputs(d1), dev_inputs(d2)
        o1 = torch.empty_like(t1["v"])
        a.forward(t1["q"], t1["k"], t1["v"], t1["a"], t1["beta"], o1)
        ckpt = a.state_get().clone()
        b.state_set(ckpt)
        oa, ob = torch.empty_like(t2["v"]), torch.empty_like(t2["v"])
        a.forward(t2["q"], t2["k"], t2["v"], t2["a"], t2["beta"], oa)
        b.forward(t2["q"], t2["k"], t2["v"], t2["a"], t2["beta"], ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob)
        assert torch.equal(a.state_get(), b.state_get())
        # and both match the oracle's carried scan
        of1, S1 = oracle.forward(d1["q"], d1["k"], d1["v"], d1["a"], d1["beta"], d1["S0"])
        of2, S2 = oracle.forward(d2["q"], d2["k"], d2["v"], d2["a"], d2["beta"], S1)
        assert_close("o chunk 2", ob, of2)
        assert_close("state", b.state_get(), S2)
    finally:
        a.close()
        b.close()


def test_repeated_calls_are_bitwise_identical():
    """No atomics or order-dependent reductions: the same call twice gives the same bits."""
    d = gdn_inputs.batch(7, 1, T1, H1, D1, with_state=True)
    t = dev_inputs(d)
    outs = []
    for _ in range(2):
        s = gb.Stream(1, H1, D1, D1, T1, poison_ws=True)
        try:
            s.state_set(torch.from_numpy(d["S0"]).cuda())
            o_f, o_r = _fwd_rev(s, t)
            outs.append((o_f, o_r, s.state_get()))
            torch.cuda.synchronize()
        finally:
            s.close()
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_no_commit_state_out_equals_commit():
    """GDN_NO_COMMIT leaves the cache as it was and writes the same final state to state_out
    that a committing call stores in the cache."""
    d = gdn_inputs.batch(8, 1, 700, 3, D1, with_state=True)
    t = dev_inputs(d)
    s = gb.Stream(1, 3, D1, D1, 700, poison_ws=True)
    try:
        S0 = torch.from_numpy(d["S0"]).cuda()
        s.state_set(S0)
        out = torch.empty_like(S0)
        o1 = torch.empty_like(t["v"])
        s.forward(t["q"], t["k"], t["v"], t["a"], t["beta"], o1, flags=gb.GDN_NO_COMMIT, state_out=out)
        assert torch.equal(s.state_get(), S0)
        o2 = torch.empty_like(t["v"])
        s.forward(t["q"], t["k"], t["v"], t["a"], t["beta"], o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert torch.equal(s.state_get(), out)
    finally:
        s.close()


def test_slow_forgetting_gates_carry():
    """Gates a = 1 - 1e-3 keep the carried state alive across whole chunks (the default gates
    forget it within ~100 tokens), so the state path is checked where it matters."""
    B, n_chunks = 1, 4
    s = gb.Stream(B, 4, D1, D1, T1, poison_ws=True)
    try:
        S_ref = None
        for c in range(n_chunks):
            d = gdn_inputs.batch(9, B, T1, 4, D1, chunk=c, with_state=(c == 0), gates="stress")
            if c == 0:
                S_ref = d["S0"].astype(np.float64)
                s.state_set(torch.from_numpy(d["S0"]).cuda())
            t = dev_inputs(d)
            o_f, o_r = _fwd_rev(s, t)
            S = s.state_get()
            torch.cuda.synchronize()
            of, S_ref = oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], S_ref)
            orv, _ = oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"])
            print(f"chunk {c}", flush=True)
            assert_close("o_fwd", o_f, of)
            assert_close("o_rev", o_r, orv)
            assert_close("state", S, S_ref)
    finally:
        s.close()
