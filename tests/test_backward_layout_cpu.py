"""CPU replica of the gradient kernels' workspace addressing (gdn_backward.hip: the state
checkpoints, the adjoint checkpoints and the row blocks' partial sums, in that order in one
allocation of backward_ws_bytes).  The address arithmetic is restated here, not imported, and
checked for what the GPU parity tests cannot see directly:

- the three regions are disjoint and inside the allocation;
- every state checkpoint the forward pass stores (one per 8-token block) and every adjoint
  checkpoint the adjoint pass stores (one per 64-token segment, at the segment's end) lies in
  its (b, h, row block)'s slice of its region;
- every checkpoint a segment walk loads was stored by phase 0 of the same call (the walk of
  segment s starts from adjoint checkpoint s and reads the state checkpoints of its blocks);
- every partial-sum row written for a token lies in the partial-sum region, and the rows of
  different (b, t, h, row block) do not overlap.
"""
import math

import numpy as np
import pytest

RB, TB, SEG = 4, 8, 64   # state rows per workgroup, tokens per staged block, tokens per segment


def layout(B, H, Dk, Dv, max_tokens):
    nrb = Dv // RB
    ck_per = math.ceil(max_tokens / TB) + 1
    gck_per = math.ceil(max_tokens / SEG)
    states = B * H * nrb * ck_per * RB * Dk
    gck = B * H * nrb * gck_per * RB * Dk
    wid = 2 * Dk + 4
    partials = B * max_tokens * H * nrb * wid
    return dict(nrb=nrb, ck_per=ck_per, gck_per=gck_per, states=states, gck=gck, wid=wid,
                total=states + gck + partials)


CASES = [(1, 20, 112, 112, 2640, 2640), (2, 3, 32, 16, 700, 300), (1, 2, 128, 128, 129, 129),
         (1, 1, 16, 16, 64, 1), (1, 2, 48, 48, 200, 65), (3, 1, 64, 32, 100, 63)]


@pytest.mark.parametrize("B, H, Dk, Dv, max_tokens, T", CASES)
def test_backward_workspace_regions(B, H, Dk, Dv, max_tokens, T):
    L = layout(B, H, Dk, Dv, max_tokens)
    nrb, wid = L["nrb"], L["wid"]
    nblk = math.ceil(T / TB)
    nseg = math.ceil(T / SEG)
    bps = SEG // TB
    ck_written, gck_written = set(), set()
    for b in range(B):
        for h in range(H):
            for rb in range(nrb):
                base_ck = ((b * H + h) * nrb + rb) * L["ck_per"] * RB * Dk
                base_gk = L["states"] + ((b * H + h) * nrb + rb) * L["gck_per"] * RB * Dk
                # phase 0, forward pass: the state before every block
                for blk in range(nblk):
                    lo = base_ck + blk * RB * Dk
                    assert base_ck <= lo and lo + RB * Dk <= base_ck + L["ck_per"] * RB * Dk
                    assert lo + RB * Dk <= L["states"]
                    ck_written.add(lo)
                # phase 0, adjoint pass: dL/dS at the end of every segment (blocks walked backward)
                for blk in range(nblk - 1, -1, -1):
                    if blk == nblk - 1 or (blk + 1) % bps == 0:
                        lo = base_gk + (blk // bps) * RB * Dk
                        assert base_gk <= lo and lo + RB * Dk <= base_gk + L["gck_per"] * RB * Dk
                        assert L["states"] <= lo and lo + RB * Dk <= L["states"] + L["gck"]
                        gck_written.add(lo)
                # phase 1: the walk of segment s reads adjoint checkpoint s and its blocks' states
                for s in range(nseg):
                    assert base_gk + s * RB * Dk in gck_written, (b, h, rb, s)
                    blo, bhi = s * bps, min(nblk, s * bps + bps) - 1
                    assert blo <= bhi
                    for blk in range(blo, bhi + 1):
                        assert base_ck + blk * RB * Dk in ck_written
    # partial-sum rows: one per (b, t, h, row block), wid floats, after both checkpoint regions
    starts = []
    for b in range(B):
        for t in range(T):
            for h in range(H):
                for rb in range(nrb):
                    off = L["states"] + L["gck"] + (((b * T + t) * H + h) * nrb + rb) * wid
                    assert off + wid <= L["total"]
                    starts.append(off)
    starts = np.sort(np.array(starts))
    assert np.all(np.diff(starts) >= wid)


def test_workspace_size_matches_the_header_formula():
    """include/gdn_stream.h: 4 (B H (d_v/4)(ceil(max_tokens/8)+1 + ceil(max_tokens/64)) 4 d_k
    + B max_tokens H (d_v/4)(2 d_k + 4)) bytes."""
    for B, H, Dk, Dv, mt, _ in CASES:
        L = layout(B, H, Dk, Dv, mt)
        hdr = B * H * (Dv // 4) * (math.ceil(mt / 8) + 1 + math.ceil(mt / 64)) * 4 * Dk + B * mt * H * (Dv // 4) * (2 * Dk + 4)
        assert L["total"] == hdr
