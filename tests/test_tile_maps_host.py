"""The GEMM tile mappings cover every tile exactly once (host logic).

The weight-gradient GEMMs hand each XCD a list of tile positions: a
contiguous range of per_xcd = ceil(total / 8) tiles, or runs of 4 tiles
dealt round-robin over the 8 XCDs.  The persistent bf16 kernel walks its
XCD's list from a counter and stops at the first position whose tile index
is past the end; the non-persistent kernels (fp32 accumulate-into, MXFP8)
take the position from the workgroup index over a grid of whole runs.  Both
forms must cover each tile index in [0, total) exactly once, whatever the
flag kernel decides.

The grouped-M GEMMs (forward and activation gradients) build their tile list
on the device: expert-major, ceil(m_e / 256) M-tiles times the N-tiles per
expert, a contiguous range of the list per XCD, and within an expert groups
of four M-tiles (N-tiles across a group, M-tiles fastest within).  Restated
here, the list must hold every (expert, M-tile, N-tile) once, its row ranges
must cover each expert's rows exactly once per N-tile, and 32 consecutive
tiles of a large expert must touch only a few M-slices.
"""
import random
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


# ---- grouped-M tile schedule ------------------------------------------------

BM = 256
GM = 4           # M-tiles per group


def grouped_tile(local, mtn, ntn, gm):
    """(mt, nt) of the local-th tile of an mtn x ntn grid walked in groups of gm M-tiles."""
    per_group = gm * ntn
    g = local // per_group
    first = g * gm
    rows = min(mtn - first, gm)
    r = local - g * per_group
    return first + r % rows, r // rows


def m_schedule(offsets, ntn, grid):
    """The tiles the workgroups of a grouped-M launch of `grid` workgroups take."""
    E = len(offsets) - 1
    m = [max(offsets[e + 1] - offsets[e], 0) for e in range(E)]
    tiles = [((me + BM - 1) // BM) * ntn for me in m]
    starts = [sum(tiles[:e]) for e in range(E)]
    total = sum(tiles)
    per_xcd = (total + XCDS - 1) // XCDS
    out = []
    for b in range(grid):
        slot, xcd = b // XCDS, b % XCDS
        if slot >= per_xcd:
            continue
        L = xcd * per_xcd + slot
        if L >= total:
            continue
        e = max(i for i in range(E) if starts[i] <= L and tiles[i] > 0)
        mt, nt = grouped_tile(L - starts[e], (m[e] + BM - 1) // BM, ntn, GM)
        row0 = offsets[e] + mt * BM
        out.append((e, mt, nt, row0, min(BM, m[e] - mt * BM)))
    return out, total


@pytest.mark.parametrize("mtn", [1, 2, 3, 4, 5, 7, 8, 9, 32, 33, 48])
@pytest.mark.parametrize("ntn", [1, 6, 12, 16])
def test_grouped_tile_is_a_bijection(mtn, ntn):
    got = Counter(grouped_tile(l, mtn, ntn, GM) for l in range(mtn * ntn))
    assert set(got) == {(a, b) for a in range(mtn) for b in range(ntn)}
    assert max(got.values()) == 1


@pytest.mark.parametrize("seed", range(6))
def test_m_schedule_covers_every_row_once(seed):
    rng = random.Random(seed)
    E = rng.choice([1, 3, 8, 16, 128])
    ntn = rng.choice([1, 6, 12, 16])
    sizes = [rng.choice([0, 1, 63, 64, 65, 255, 256, 257, 513, 2048 + 7, 8192]) for _ in range(E)]
    offsets = [0]
    for n in sizes:
        offsets.append(offsets[-1] + n)
    n_rows = offsets[-1]
    grid = ((n_rows // BM + E) * ntn + XCDS - 1) // XCDS * XCDS   # the host's bound
    out, total = m_schedule(offsets, ntn, grid)
    assert len(out) == total == len({t[:3] for t in out})
    for nt in range(ntn):
        covered = Counter()
        for e, mt, t_nt, row0, valid in out:
            if t_nt == nt:
                assert 0 < valid <= BM
                covered.update(range(row0, row0 + valid))
        assert set(covered) == set(range(n_rows)) and (not covered or max(covered.values()) == 1)


def test_m_schedule_groups_m_tiles_of_a_large_expert():
    # one 8192-row expert (32 M-tiles) x 12 N-tiles: 32 consecutive tiles (an
    # XCD's workgroups at once) read at most two groups' M-slices, not 32
    mtn, ntn = 32, 12
    order = [grouped_tile(l, mtn, ntn, GM) for l in range(mtn * ntn)]
    for w in range(0, mtn * ntn - 32):
        assert len({mt for mt, _ in order[w:w + 32]}) <= 2 * GM
