"""Oracle of the low-precision projection GEMMs of the GDN block (test infrastructure only).

The pages' mixed-precision quantisation (the Chinese summary, "Results", Table 2 and Figure 6; the Korean review,
section 1 "Key Terms", MPQ) runs the block's projections as FP8 / FP4 GEMMs; they print neither the formats' details
nor the scaling policy.  Readings taken here:

- FP8 is OCP E4M3: sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  m * 2^-9; S.1111.111 is NaN and there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
  Conversion rounds to nearest with ties to even and saturates at +-448 (the "satfinite" conversion).
- Activations are scaled per row (token) and weights per row (output feature).  The stored dequantisation scale is
  s = amax / 448 and the codes are E4M3(x * r) with r = 448 / amax, both divisions IEEE float32 (correctly rounded)
  and the product a float32 multiply, so the integer codes are a float32 decision taken identically on both sides
  (one division per row rather than per element); a row of zeros gets s = 0 and codes 0.
- The GEMM: C[i][j] = sa[i] * sw[j] * sum_k E4M3^-1(A[i][k]) * E4M3^-1(W[j][k]), accumulated in float32 by the
  kernel (every product of two E4M3 values is exact in float32) and stored as bfloat16 (round to nearest even); here
  the sum is exact in float64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of every E4M3 code 0..255 (float64; NaN for S.1111.111), from the format's definition."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DEC = e4m3_decode_table()
# the finite non-negative codes in increasing order of value (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = _DEC[_POS_CODES]


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3 codes: nearest representable value, ties to the even code (the one whose lowest
    mantissa bit is 0), magnitudes beyond 448 saturate to 448, NaN is not expected.  Vectorised by bracketing each
    magnitude between consecutive representable values."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALS, mag, side="left")          # first value >= mag
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _POS_VALS[lo], _POS_VALS[hi]
    exact = vhi == mag
    dlo, dhi = mag - vlo, vhi - mag
    pick_hi = exact | (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(mag == 0.0, 0, code)
    sign = (x < 0) & (code != 0)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _DEC[np.asarray(codes, dtype=np.int64)]


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3 quantisation of a 2-D array: (codes uint8 [rows, cols], scales float32 [rows]).  The scale s,
    the code multiplier r and the scaled values are float32 computations, as the kernel does them."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    nz = amax > 0
    r = np.where(nz, np.float32(E4M3_MAX) / np.where(nz, amax, np.float32(1)), np.float32(0)).astype(np.float32)
    y = (x32 * r[:, None]).astype(np.float32)
    return e4m3_encode(y), s


def gemm_e4m3(a_codes, a_scales, w_codes, w_scales) -> np.ndarray:
    """C = diag(sa) dec(A) dec(W)^T diag(sw) in float64 (exact up to the float64 sum of exact products)."""
    a = e4m3_decode(a_codes)
    w = e4m3_decode(w_codes)
    return (np.asarray(a_scales, np.float64)[:, None] * (a @ w.T)) * np.asarray(w_scales, np.float64)[None, :]


def bf16_round(x) -> np.ndarray:
    """Round float64 values to bfloat16 (via float32, round to nearest even on the upper 16 bits), as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
