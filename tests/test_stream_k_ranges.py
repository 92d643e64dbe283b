"""Index arithmetic of the stream-K up projection (host-side check, no GPU).

The kernel splits T = tiles x KBT input blocks into G' = min(G, 2 x tiles) equal ranges
(range g = [g T / G', (g + 1) T / G')), finds the owner of block j as
((j + 1) G' - 1) / T, holds at most 3 parts per tile and lists at most 16 tiles per range;
the dispatcher takes it at 17-32 tokens with d a multiple of 512 (KBT = d / 512 >= 2) and
G = g_sk with 13 g_sk >= ceil(n / 16). These bounds are what the kernel's fixed-size
buffers rely on; this test walks the whole parameter space the dispatcher allows for
small grids and spot-checks large ones."""
import itertools

import pytest

SK_TMAX, SK_PMAX = 16, 3


def ranges(ntiles, KBT, grid):
    G = min(grid, 2 * ntiles)
    T = ntiles * KBT
    start = [g * T // G for g in range(G + 1)]
    return G, T, start


def owner(j, G, T):
    return ((j + 1) * G - 1) // T


def check(ntiles, KBT, grid):
    G, T, start = ranges(ntiles, KBT, grid)
    for g in range(G):
        j0, j1 = start[g], start[g + 1]
        assert j1 > j0, "every range holds at least one block"
        assert (j1 - 1) // KBT - j0 // KBT + 1 <= SK_TMAX, "tiles one range touches"
        for j in (j0, j1 - 1):
            assert owner(j, G, T) == g
    slot_tile = {}
    for t in range(ntiles):
        tb = t * KBT
        glo, ghi = owner(tb, G, T), owner(tb + KBT - 1, G, T)
        assert 1 <= ghi - glo + 1 <= SK_PMAX
        if glo == ghi:
            continue  # finished inside one range, no part published
        # each part's slot: 2g for the tile its range starts in, 2g + 1 for the one it ends
        # in; no slot may serve two tiles
        for g in range(glo, ghi + 1):
            slot = 2 * g + (0 if start[g] >= tb else 1)
            assert slot_tile.setdefault(slot, t) == t


@pytest.mark.parametrize("KBT", [2, 3, 4, 5, 6, 8, 24])
def test_small_grids_exhaustive(KBT):
    for grid, ntiles in itertools.product(range(1, 40), range(1, 200)):
        if 13 * grid >= ntiles:  # the dispatcher's bound on the grid
            check(ntiles, KBT, grid)


def test_dispatched_shapes():
    # grids of two workgroups per compute unit (up to 512) over lists of every size the
    # library takes (n <= 65536, so up to 4096 16-row tiles)
    for grid in (256, 304, 512):
        for KBT in (2, 8, 24):
            for ntiles in list(range(1, 300)) + list(range(300, 4097, 37)):
                if 13 * grid >= ntiles:
                    check(ntiles, KBT, grid)


def test_owner_matches_ranges():
    for T, G in itertools.product(range(1, 300), range(1, 64)):
        if G > T:
            continue
        start = [g * T // G for g in range(G + 1)]
        for j in range(T):
            g = owner(j, G, T)
            assert start[g] <= j < start[g + 1]
