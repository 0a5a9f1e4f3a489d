"""The weight-gradient tile mappings cover every tile exactly once (host logic).

The weight-gradient GEMMs hand each XCD a list of tile positions: a
contiguous range of per_xcd = ceil(total / 8) tiles, or runs of 4 tiles
dealt round-robin over the 8 XCDs.  The persistent bf16 kernel walks its
XCD's list from a counter and stops at the first position whose tile index
is past the end; the non-persistent kernels (fp32 accumulate-into, MXFP8)
take the position from the workgroup index over a grid of whole runs.  Both
forms must cover each tile index in [0, total) exactly once, whatever the
flag kernel decides.
"""
from collections import Counter

import pytest

RUN = 4          # tiles per dealt run
XCDS = 8


def tile_at(j, xcd, total, deal):
    """Tile index at position j of an XCD's list (total past its end)."""
    per_xcd = (total + XCDS - 1) // XCDS
    if deal:
        L = ((j // RUN) * XCDS + xcd) * RUN + j % RUN
    else:
        L = xcd * per_xcd + j if j < per_xcd else total
    return min(L, total)


def persistent_walk(total, deal):
    seen = Counter()
    for xcd in range(XCDS):
        j = 0
        while True:
            L = tile_at(j, xcd, total, deal)
            if L >= total:
                break
            seen[L] += 1
            j += 1
        # the list is increasing, so nothing lies past the first tile at the end
        assert all(tile_at(jj, xcd, total, deal) >= total for jj in range(j, j + 3 * RUN * XCDS))
    return seen


def grid_walk(total, deal):
    grid = (total + XCDS * RUN - 1) // (XCDS * RUN) * (XCDS * RUN)
    seen = Counter()
    for b in range(grid):
        L = tile_at(b // XCDS, b % XCDS, total, deal)
        if L < total:
            seen[L] += 1
    return seen


@pytest.mark.parametrize("deal", [False, True])
@pytest.mark.parametrize("total", [1, 7, 8, 31, 32, 33, 100, 288 * 3, 288 * 128, 288 * 128 + 17, 12345])
def test_each_tile_exactly_once(total, deal):
    for walk in (persistent_walk, grid_walk):
        seen = walk(total, deal)
        assert set(seen) == set(range(total)), (walk.__name__, total, deal)
        assert max(seen.values()) == 1, (walk.__name__, total, deal)


def test_dealt_runs_spread_a_group_over_all_xcds():
    # the point of dealing: the tiles of one group (here 288 consecutive tile
    # indices) land on every XCD, in runs of 4
    total = 288 * 16
    owner = {}
    for xcd in range(XCDS):
        j = 0
        while (L := tile_at(j, xcd, total, True)) < total:
            owner[L] = xcd
            j += 1
    for g in range(16):
        assert {owner[L] for L in range(288 * g, 288 * (g + 1))} == set(range(XCDS))
        for L in range(288 * g, 288 * (g + 1), RUN):
            assert len({owner[L + r] for r in range(RUN) if L + r < 288 * (g + 1)}) == 1
