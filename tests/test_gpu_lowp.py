"""GPU parity of the FP8 (E4M3) projection GEMMs through the C ABI against oracle/lowp_gemm.py.

Quantisation is an integer decision taken in float32 on both sides, so codes and scales must match bit for
bit.  The GEMM sums exact products in float32 and rounds to bf16: the bar per element is
|y - ref| <= 2^-8 |ref| + K 2^-24 s_x s_w sum_k |x_k w_k|, the bf16 rounding (half an ulp, 2^-9, with a factor 2
for the two float32 scale products) plus the standard bound (K - 1) u of a float32 sum of K terms.
The oracle quantises its own inputs; nothing it compares with comes from the GPU.
"""
import numpy as np
import pytest

import gdn_inputs
from oracle import lowp_gemm as lg

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from gated_deltanet_streaming_amd import binding as gb  # noqa: E402


def _dev(a, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dtype)


def _check_gemm(y, xq, xs, wq, ws, rows=None):
    ref = lg.gemm_e4m3(xq if rows is None else xq[rows], xs if rows is None else xs[rows], wq, ws)
    a = np.abs(lg.e4m3_decode(xq if rows is None else xq[rows]))
    K = xq.shape[1]
    bound = np.abs(ref) * 2.0 ** -8 + K * 2.0 ** -24 * (np.asarray(xs if rows is None else xs[rows])[:, None]
                                                     * (a @ np.abs(lg.e4m3_decode(wq)).T) * np.asarray(ws)[None, :])
    got = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    err = np.abs(got - ref)
    print(f"  max |err| {err.max():.3e}, max |ref| {np.abs(ref).max():.3e}, worst err/bound {np.max(err / np.maximum(bound, 1e-30)):.3f}",
          flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_rows_bit_exact(dtype):
    x, _ = gdn_inputs.proj_inputs(81, 300, 2240, 4)
    x[5] = 0.0                         # a zero row
    x[6] *= 1e3                        # large magnitudes
    x[7] *= 1e-6                       # tiny ones: subnormal codes
    x[8, :7] = [448.0, -448.0, 1.0625, -2.0 ** -10, 3.0, 1e-30, -0.0]
    if dtype == "bf16":
        x = gdn_inputs.round_bf16(x)
    xd = _dev(x, torch.bfloat16 if dtype == "bf16" else torch.float32)
    print(f"quantize {dtype}: rows 300 cols 2240", flush=True)
    codes, scales = gb.quantize_rows_e4m3(xd)
    torch.cuda.synchronize()
    rq, rs = lg.quantize_rows(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != rq)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}: {got[tuple(bad[0])]:#x} vs {rq[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("rows, cols, offset", [(37, 2243, 0), (9, 5000, 0), (11, 4096, 0), (13, 2240, 1), (5, 8, 0)])
def test_quantize_rows_every_path(rows, cols, offset):
    """Ragged widths, rows wider than the register-resident form, a misaligned view (general form) and the
    widest and narrowest rows of the vector form: codes and scales bit-exact against the oracle."""
    x, _ = gdn_inputs.proj_inputs(84, rows, cols + offset, 4)
    x = gdn_inputs.round_bf16(x)
    print(f"quantize rows {rows} cols {cols} offset {offset}", flush=True)
    xd = _dev(x)[:, offset:]
    codes, scales = gb.quantize_rows_e4m3(xd)
    torch.cuda.synchronize()
    rq, rs = lg.quantize_rows(x[:, offset:])
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rq)


# shapes chosen so that, on 256 compute units, the host picks each workgroup tile (features x tokens): 128 x 128
# (the small ones), 256 x 128 (2048 x 4096, two bands of token tiles), 192 x 128 (128 x 49152, and the 720p
# projection below) and 192 x 192 (384 x 24576); K spans one step, a ragged last step, and many steps
@pytest.mark.parametrize("M, N, K", [(200, 136, 272), (1, 4, 16), (129, 260, 2240), (64, 128, 128), (2048, 4096, 1040),
                                     (128, 49152, 256), (384, 24576, 256)])
def test_gemm_matches_the_oracle(M, N, K):
    x, w = gdn_inputs.proj_inputs(82, M, K, N)
    xq, xs = lg.quantize_rows(x)
    wq, ws = lg.quantize_rows(w)
    print(f"gemm M {M} N {N} K {K}", flush=True)
    gxq, gxs = gb.quantize_rows_e4m3(_dev(x))
    gwq, gws = gb.quantize_rows_e4m3(_dev(w))
    y = gb.gemm_e4m3(gxq, gxs, gwq, gws)
    torch.cuda.synchronize()
    _check_gemm(y, xq, xs, wq, ws)


def test_gemm_720p_projection_sampled_rows():
    """The fused q/k/v projection of one GDN block at the 720p chunk: 2640 tokens x 2240 -> 6720, every column of
    48 sampled token rows (first, last, tile edges and random) against the oracle."""
    M, K, N = 2640, 2240, 6720
    x, w = gdn_inputs.proj_inputs(83, M, K, N)
    print(f"gemm 720p M {M} N {N} K {K}", flush=True)
    gxq, gxs = gb.quantize_rows_e4m3(_dev(x))
    gwq, gws = gb.quantize_rows_e4m3(_dev(w))
    y = gb.gemm_e4m3(gxq, gxs, gwq, gws)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 2559, 2560, M - 1],
                                     np.random.default_rng(83).choice(M, 41, replace=False)]))
    xq, xs = lg.quantize_rows(x[rows])
    wq, ws = lg.quantize_rows(w)
    # quantisation of the sampled rows is bit-exact on both sides (checked above); compare the GEMM rows
    assert np.array_equal(gxq.cpu().numpy()[rows], xq) and np.array_equal(gxs.cpu().numpy()[rows], xs)
    ref_y = y[torch.from_numpy(rows).cuda()]
    _check_gemm(ref_y, xq, xs, wq, ws)


def test_gemm_zero_k_and_empty_shapes():
    # K = 0 through views of real buffers (an empty tensor may have no storage)
    xq = torch.zeros((8, 16), dtype=torch.uint8, device="cuda")[:, :0]
    wq = torch.zeros((4, 16), dtype=torch.uint8, device="cuda")[:, :0]
    s8 = torch.ones(8, dtype=torch.float32, device="cuda")
    s4 = torch.ones(4, dtype=torch.float32, device="cuda")
    y = torch.full((8, 8), 5.0, dtype=torch.bfloat16, device="cuda")[:, :4]
    gb.gemm_e4m3(xq, s8, wq, s4, y)
    torch.cuda.synchronize()
    assert bool((y == 0).all())
    e = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    gb.gemm_e4m3(e, s8[:0], torch.zeros((4, 16), dtype=torch.uint8, device="cuda"), s4)


def test_gemm_is_bitwise_repeatable():
    x, w = gdn_inputs.proj_inputs(84, 300, 512, 260)
    gxq, gxs = gb.quantize_rows_e4m3(_dev(x))
    gwq, gws = gb.quantize_rows_e4m3(_dev(w))
    y1 = gb.gemm_e4m3(gxq, gxs, gwq, gws)
    y2 = gb.gemm_e4m3(gxq, gxs, gwq, gws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
