"""GPU parity of the softmax block's sink + window attention (include/gdn_attn.h) against the
fp64 oracle (oracle/window_attn.py), through the C ABI.

Every call of a stream is compared element by element with the oracle on the same seeded
bf16 inputs, at max-abs <= 2e-2 and relative Frobenius <= 5e-3 over the call's output.  Cases:
ragged chunks that cross the 64-key tile and 32-query wavefront boundaries, a sink that
fills over two calls, chunks longer than the window, no sink, no window, no cache at all,
uncommitted replays (bitwise repeatable, cache unchanged), peaked logits, strided [B, H, T, D]
buffers, and the 720p layer shape (20 heads x 112, one latent frame of sink, one chunk of
window) through three chunks to the steady state, checked on sampled query rows; and a cache
checkpoint restored into a second handle, which then continues bitwise identically.
"""
import numpy as np
import pytest

import gdn_inputs
from oracle.window_attn import SinkWindowAttention
from tests.gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _dev(x, layout="bthd"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    if layout == "bhtd":
        return t.permute(0, 2, 1, 3).contiguous().to("cuda", torch.bfloat16).permute(0, 2, 1, 3)
    return t.to("cuda", torch.bfloat16)


def _run_stream(D, n_sink, n_window, sizes, *, B=2, H=3, commits=None, q_scale=1.0, layout="bthd", seed=0):
    import torch
    from gated_deltanet_streaming_amd.binding import WindowAttention
    att = WindowAttention(B, H, D, n_sink, n_window, max(sizes))
    ref = SinkWindowAttention(n_sink, n_window)
    commits = commits or [True] * len(sizes)
    for c, (T, commit) in enumerate(zip(sizes, commits)):
        d = gdn_inputs.attn_chunk(c, B, T, H, D, stream=seed, q_scale=q_scale)
        q, k, v = (_dev(d[x], layout) for x in ("q", "k", "v"))
        o = torch.empty_like(v)
        print(f"case D={D} sink={n_sink} window={n_window} call={c} T={T} commit={commit}", flush=True)
        att.chunk(q, k, v, o, commit=commit)
        torch.cuda.synchronize()
        want = ref.chunk(d["q"], d["k"], d["v"], commit=commit)
        assert_close(f"o[{c}]", o, want)
        hist = ref.history
        assert att.cache_len() == (min(hist, n_sink), min(max(hist - n_sink, 0), n_window))
    att.close()


@pytest.mark.parametrize("D", [64, 112, 128])
def test_ragged_stream(D):
    # sink fills over the first two calls; the 200-token chunk is longer than the window
    _run_stream(D, 40, 100, [30, 130, 5, 200, 64, 129])


def test_no_sink_no_window():
    _run_stream(112, 0, 0, [150, 70])


def test_window_only_and_sink_only():
    _run_stream(112, 0, 96, [64, 64, 64])
    _run_stream(112, 80, 0, [50, 60, 70])


def test_uncommitted_replay_is_bitwise_and_keeps_the_cache():
    import torch
    from gated_deltanet_streaming_amd.binding import WindowAttention
    B, H, D, T = 1, 4, 112, 300
    att = WindowAttention(B, H, D, 64, 256, T)
    d0 = gdn_inputs.attn_chunk(0, B, T, H, D)
    att.chunk(*(_dev(d0[x]) for x in ("q", "k", "v")))
    before = att.cache_len()
    d1 = gdn_inputs.attn_chunk(1, B, T, H, D)
    q, k, v = (_dev(d1[x]) for x in ("q", "k", "v"))
    a = att.chunk(q, k, v, commit=False)
    b = att.chunk(q, k, v, commit=False)
    torch.cuda.synchronize()
    assert att.cache_len() == before
    assert torch.equal(a, b)
    c = att.chunk(q, k, v, commit=True)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
    att.close()


def test_peaked_logits():
    _run_stream(112, 32, 128, [100, 100, 100], q_scale=4.0, seed=3)


def test_strided_bhtd_buffers():
    _run_stream(112, 16, 64, [77, 90], layout="bhtd", seed=5)


def test_zero_tokens_is_a_no_op():
    import torch
    from gated_deltanet_streaming_amd.binding import WindowAttention
    att = WindowAttention(1, 2, 64, 8, 8, 16)
    x = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    att.chunk(x, x, x, x)
    assert att.cache_len() == (0, 0)
    att.close()


def test_720p_layer_steady_state_sampled_rows():
    """B=1, H=20, d=112, sink = one latent frame (880 tokens), window = one chunk (2640), three
    chunks of 2640: the third attends over 880 + 2640 + 2640 = 6160 keys."""
    import torch
    from gated_deltanet_streaming_amd.binding import WindowAttention
    B, H, D, T = 1, 20, 112, 2640
    att = WindowAttention(B, H, D, 880, 2640, T)
    ref = SinkWindowAttention(880, 2640)
    rows = np.sort(np.random.default_rng(0).choice(T, 192, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 63, 64, 127, 128, T - 1]]))
    for c in range(3):
        d = gdn_inputs.attn_chunk(c, B, T, H, D)
        q, k, v = (_dev(d[x]) for x in ("q", "k", "v"))
        print(f"case 720p call={c}", flush=True)
        o = att.chunk(q, k, v)
        torch.cuda.synchronize()
        want = ref.chunk(d["q"][:, rows], d["k"], d["v"])
        assert_close(f"o[{c}] rows", o[:, torch.from_numpy(rows).cuda()], want)
    assert att.cache_len() == (880, 2640)
    att.close()


def test_720p_layer_steady_state_every_row_of_two_heads():
    """The same 720p steady state (third chunk: 6160 keys), every one of the 2640 query rows of
    heads 0 and 13 against the reference fed those heads' q, k, v for all three chunks (heads
    are independent)."""
    import torch
    from gated_deltanet_streaming_amd.binding import WindowAttention
    B, H, D, T = 1, 20, 112, 2640
    heads = [0, 13]
    att = WindowAttention(B, H, D, 880, 2640, T)
    ref = SinkWindowAttention(880, 2640)
    for c in range(3):
        d = gdn_inputs.attn_chunk(c, B, T, H, D)
        q, k, v = (_dev(d[x]) for x in ("q", "k", "v"))
        print(f"case 720p every row, heads {heads}, call={c}", flush=True)
        o = att.chunk(q, k, v)
        torch.cuda.synchronize()
        want = ref.chunk(d["q"][:, :, heads], d["k"][:, :, heads], d["v"][:, :, heads])
        assert_close(f"o[{c}] heads {heads}", o[:, :, heads], want)
    att.close()


def test_checkpoint_resume_is_bitwise():
    """A handle resumed from another's cache snapshot continues bitwise identically; bad
    counters are refused."""
    import torch
    from gated_deltanet_streaming_amd.binding import GdnError, WindowAttention
    B, H, D = 2, 3, 112
    a = WindowAttention(B, H, D, 40, 100, 130)
    for c, T in enumerate((30, 130, 64)):
        d = gdn_inputs.attn_chunk(c, B, T, H, D)
        a.chunk(*(_dev(d[x]) for x in ("q", "k", "v")))
    snap, s_len, w_tot = a.checkpoint()
    assert (s_len, w_tot) == (40, 184)
    b = WindowAttention(B, H, D, 40, 100, 130)
    with pytest.raises(GdnError):
        b.restore(snap, 10, 5)          # a window cannot fill before the sink
    b.restore(snap, s_len, w_tot)
    assert b.cache_len() == a.cache_len()
    d = gdn_inputs.attn_chunk(3, B, 120, H, D)
    x = [_dev(d[k]) for k in ("q", "k", "v")]
    oa, ob = a.chunk(*x), b.chunk(*x)
    d = gdn_inputs.attn_chunk(4, B, 50, H, D)
    x = [_dev(d[k]) for k in ("q", "k", "v")]
    oa2, ob2 = a.chunk(*x), b.chunk(*x)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(oa2, ob2)
    a.close()
    b.close()
