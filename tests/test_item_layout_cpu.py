"""CPU replica of the chunked path's workspace addressing: where the prep kernel stores each
item byte and where the scan kernel reads it back (gdn_kernels.hip, prep item stores and the
scan's item loads).  The kernels' address arithmetic is restated here, not imported, and
checked for the properties the parity tests cannot see directly:

- the items of (direction, stream, head, sub-chunk) are disjoint and inside the workspace;
- every prep store of a block lands inside its own item;
- every item byte the scan uses was stored by the prep of the same call (a byte it did not
  store would be whatever the workspace held before: NaN under GDN_POISON_WS);
- every scan load of an item lies inside its buffer resource (base = the first item of the
  (direction, stream, head), num_records = N items): a load past num_records returns zero,
  which poisoning cannot reveal;
- the scan's step n of either direction reads the item the prep wrote for that step, and the
  output wavefronts' lane-major c2 reads find the scalar of the token they scale.
"""
import numpy as np
import pytest


def blocks(NB):
    """Row tile mt of a C x C lower-triangular operand needs count(mt) fragments (32-wide
    k-steps reaching its diagonal, plus a trailing 16-wide one when NB is odd)."""
    nfull = NB // 2
    half = NB % 2 == 1
    count = [min(mt // 2 + 1, nfull) + (1 if half and mt == NB - 1 else 0) for mt in range(NB)]
    offset = np.concatenate([[0], np.cumsum(count)]).astype(int)
    return count, offset


def out_tiles(NB):
    """Token tiles of each output wavefront: two wavefronts when NB >= 2; with two tiles each,
    wavefront O takes tiles O and NB - 1 - O."""
    nout = 2 if NB >= 2 else 1
    tpo = NB // nout
    if tpo == 2:
        return [[O, NB - 1 - O] for O in range(nout)]
    return [[O * tpo + t for t in range(tpo)] for O in range(nout)]


def layout(C, B, H, T, nsub_max):
    NB = C // 16
    count, offset = blocks(NB)
    NF = int(offset[-1])
    ib = 1024 * (2 * NF + 1)
    N = (T + C - 1) // C
    ws = 2 * B * H * nsub_max * ib
    return dict(NB=NB, count=count, offset=offset, NF=NF, ib=ib, N=N, ws=ws, nsub_max=nsub_max, sc=2 * NF * 1024)


def item_base(L, B, H, d, b, h, n):
    return ((((d * B) + b) * H + h) * L["nsub_max"] + n) * L["ib"]


def prep_stores(L, C, d, j):
    """Byte ranges (start, length) within the item that the prep block j stores for direction d,
    and the item index it stores them in."""
    N, NF, sc = L["N"], L["NF"], L["sc"]
    n = N - 1 - j if d else j
    out = []
    for kind in (0, 1):                       # T~ fragments, then A^T fragments
        for f in range(NF):
            for lane in range(64):
                out.append(((kind * NF + f) * 1024 + 16 * lane, 16))
    NB = L["NB"]
    for pr in range(C):                       # processing row pr: c1, w, c2 (lane-major), gamma_C
        out.append((sc + 4 * pr, 4))
        out.append((sc + 4 * (C + pr), 4))
        out.append((sc + 4 * (2 * C + (pr & 15) * NB + (pr >> 4)), 4))
    out.append((sc + 4 * 3 * C, 4))
    return n, out


def scan_item_reads(L, C):
    """For step n: (voffset, soffset, length, used) of every item load the scan makes, relative to
    the first item of the (direction, stream, head); `used` is the number of leading bytes of the
    load the kernel computes with (the 1 KB scalar block is loaded whole but only its 3C + 1
    scalars are used)."""
    NB, NF, ib, sc, count, offset = L["NB"], L["NF"], L["ib"], L["sc"], L["count"], L["offset"]
    reads = []
    for n in range(L["N"]):
        soff = n * ib
        for f in range(NF):                               # loader: T~ fragments into LDS
            for lane in range(64):
                reads.append((1024 * f + 16 * lane, soff, 16, 16))
        for lane in range(64):                            # loader: the scalar block
            lo = 16 * lane
            reads.append((sc + lo, soff, 16, min(16, max(0, 4 * (3 * C + 1) - lo))))
        for O, tiles in enumerate(out_tiles(NB)):         # output wavefronts
            for tile in tiles:
                for kt in range(count[tile]):
                    for lane in range(64):
                        reads.append((16 * lane, soff + 1024 * (NF + offset[tile] + kt), 16, 16))
                for r in range(16):
                    reads.append((4 * (NB * r + tile), soff + sc + 8 * C, 4, 4))
    return reads


CASES = [(C, B, H, T, nsub_extra) for C in (16, 32, 64)
         for (B, H, T, nsub_extra) in ((2, 3, 600, 0), (2, 3, 700, 0), (1, 20, 2640, 0), (1, 4, 150, 3), (1, 2, 1, 0))]


@pytest.mark.parametrize("C, B, H, T, nsub_extra", CASES)
def test_items_are_written_before_they_are_read(C, B, H, T, nsub_extra):
    N = (T + C - 1) // C
    L = layout(C, B, H, T, N + nsub_extra)     # a handle sized for more tokens than this call
    ib, ws = L["ib"], L["ws"]
    # items are disjoint and inside the workspace
    bases = sorted(item_base(L, B, H, d, b, h, n) for d in (0, 1) for b in range(B) for h in range(H)
                   for n in range(L["nsub_max"]))
    assert bases[0] == 0 and bases[-1] + ib <= ws
    assert all(y - x == ib for x, y in zip(bases, bases[1:]))

    written = np.zeros(ws, dtype=np.int32)
    for d in (0, 1):
        for b in range(B):
            for h in range(H):
                for j in range(N):
                    n, stores = prep_stores(L, C, d, j)
                    assert 0 <= n < N
                    base = item_base(L, B, H, d, b, h, n)
                    for off, ln in stores:
                        assert 0 <= off and off + ln <= ib, (d, b, h, j, off)
                        written[base + off:base + off + ln] += 1
    # each item of the call is stored once (by one block), the c2 scatter is a permutation
    for d in (0, 1):
        for b in range(B):
            for h in range(H):
                for n in range(N):
                    base = item_base(L, B, H, d, b, h, n)
                    w = written[base:base + ib]
                    assert w.max() <= 1, "two stores to one byte"
                    assert w[:2 * L["NF"] * 1024].all()
                    assert w[L["sc"]:L["sc"] + 4 * (3 * C + 1)].all()

    reads = scan_item_reads(L, C)
    num_records = N * ib
    for d in (0, 1):
        for b in range(B):
            for h in range(H):
                item0 = item_base(L, B, H, d, b, h, 0)
                for voff, soff, ln, used in reads:
                    # inside the resource whether or not the hardware counts soffset in the check
                    assert voff + ln <= num_records and voff + soff + ln <= num_records
                    a = item0 + soff + voff
                    assert written[a:a + used].all(), (d, b, h, soff // ib, voff)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_c2_lane_major_order_matches_the_output_reads(C):
    """The prep stores token pr's c2 at 2C + (pr % 16) NB + pr // 16; the output wavefront that
    scales token 16 tile + r reads 2C + NB r + tile."""
    NB = C // 16
    for tile in range(NB):
        for r in range(16):
            pr = 16 * tile + r
            assert 2 * C + (pr & 15) * NB + (pr >> 4) == 2 * C + NB * r + tile


def test_every_token_tile_has_one_output_wavefront():
    for NB in (1, 2, 3, 4, 5):
        tiles = sorted(t for ts in out_tiles(NB) for t in ts)
        if NB % 2 == 0 or NB == 1:
            assert tiles == list(range(NB)), NB
