"""Address bounds of the attention kernels' K and V^T tile copies, computed on
the host from the same index formulas the kernels use (no device code runs).

Each K tile travels global -> LDS through a buffer descriptor that starts at the
tile and whose num_records is the byte count from there to the end of the
head's K; lanes read at per-lane byte offsets with a zero scalar offset.  The
hardware's per-lane range check compares the lane offset with num_records and
returns zeros past it.  These tests show, for the ragged last tile of the last
head at every shape tried, that the lanes inside the range are exactly the key
rows below seq_len and read only bytes of that head's K, and that every
(row, chunk) of the tile is filled exactly once.  V^T tiles are zero-padded
whole blocks, so all their reads lie inside the head's transposed V.
"""
import numpy as np
import pytest

BLK = 64


def key_of_row(r):
    return (r & ~12) | ((r >> 1) & 4) | ((r << 1) & 8)


def k_swz(D, r):
    return r & 15 if D == 128 else (r >> 1) & 7


def v_swz(d):
    return (d >> 1) & 7


def k_lane_offsets(D):
    """(LDS row, LDS chunk position, byte offset in the tile) of every K copy lane."""
    CPR, KR, NI = D // 8, 1024 // (2 * D), D // 32
    out = []
    for wave in range(4):
        for i in range(NI):
            ii = wave * NI + i
            for lane in range(64):
                r = ii * KR + lane // CPR
                pos = lane % CPR
                voff = (key_of_row(r) * CPR + (pos ^ k_swz(D, r))) * 16
                out.append((r, pos, voff))
    return out


def v_lane_offsets(D, npad):
    NI = D // 32
    out = []
    for wave in range(4):
        for i in range(NI):
            ii = wave * NI + i
            for lane in range(64):
                d = 8 * ii + (lane >> 3)
                out.append((d, lane & 7, d * npad * 2 + 16 * ((lane & 7) ^ v_swz(d))))
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,N", [(40, 75600), (12, 32760), (24, 126720), (3, 1), (2, 65), (1, 64 * 7 + 5), (5, 127)])
def test_last_k_tile_reads_stay_inside_the_tensor(D, H, N):
    nb = -(-N // BLK)
    kvb = nb - 1
    head_bytes = N * D * 2
    tile_base = kvb * BLK * D * 2                      # descriptor base, relative to the head
    nrec = (N - kvb * BLK) * D * 2                     # its num_records
    rem = N - kvb * BLK                                # real keys in the tile
    lanes = k_lane_offsets(D)
    filled = np.zeros((BLK, D // 8), int)
    max_end = 0
    for r, pos, voff in lanes:
        filled[r, pos] += 1
        key = voff // (D * 2)
        in_range = voff + 16 <= nrec
        assert in_range == (key < rem)                 # exactly the real keys are read
        assert voff % 16 == 0 and (voff + 16 <= nrec or voff >= nrec)   # no 16-byte read straddles the end
        if in_range:
            max_end = max(max_end, tile_base + voff + 16)
    assert np.all(filled == 1)
    assert max_end <= head_bytes
    # the last head ends where the tensor does
    assert (H - 1) * head_bytes + max_end <= H * head_bytes
    if rem == BLK:
        assert max_end == head_bytes


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [75600, 126720, 1, 65])
def test_v_transposed_tiles_lie_inside_the_head(D, N):
    nb = -(-N // BLK)
    npad = nb * BLK
    nrec = D * npad * 2
    lanes = v_lane_offsets(D, npad)
    seen = {(d, c) for d, c, _ in lanes}
    assert len(seen) == D * 8 == len(lanes)
    worst = max(voff for _, _, voff in lanes) + (nb - 1) * BLK * 2 + 16
    assert worst <= nrec
