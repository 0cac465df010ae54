"""Host replica of the grouped GEMMs' work assignment (the schedule kernel's
row-tile counts and work_of_block in csrc/gemm_sched.hpp), checked on the
CPU: for any expert row counts, column-tile count and grid at least the item
count, and for any order in which blocks reach the shared pool's counter,
every (column tile, row) of every expert is computed exactly once, full row
tiles have more than half_rows rows and short ones at most half_rows.  The
GPU parity tests check the device code itself; this pins the arithmetic of
the assignment over many more shapes than they can run."""
import random

import pytest

GROUP = 4          # kGroup
BM, HALF = 256, 128


def row_tiles(lens, bm, half):
    """schedule_kernel: full and short row tiles per expert, exclusive prefixes."""
    fp, hp = [0], [0]
    for n in lens:
        nrt = (n + bm - 1) // bm
        h = 1 if nrt > 0 and n - (nrt - 1) * bm <= half else 0
        fp.append(fp[-1] + nrt - h)
        hp.append(hp[-1] + h)
    return fp, hp


def decode(L, fp, hp, ntn, lens, starts, bm):
    """Item L -> (expert, column tiles, first row, rows) as work_of_block."""
    npairs = (ntn + 1) >> 1
    before = lambda e: fp[e] * ntn + hp[e] * npairs
    lo, hi = 0, len(lens)
    while hi - lo > 1:
        mid = (lo + hi) >> 1
        if before(mid) <= L:
            lo = mid
        else:
            hi = mid
    e = lo
    i = L - before(e)
    F, Hs = fp[e + 1] - fp[e], hp[e + 1] - hp[e]
    nfg = max(1, (F + GROUP - 1) // GROUP)
    g = min(i // (GROUP * ntn), nfg - 1)
    i -= g * GROUP * ntn
    f = min(GROUP, F - g * GROUP)
    h = Hs if g == nfg - 1 else 0
    bs = 2 * f + h
    p = min(i // bs, npairs - 1)
    j = i - p * bs
    ncols = 2 if 2 * p + 1 < ntn else 1
    if j < f * ncols:
        mt = g * GROUP + j % f
        return e, [2 * p + j // f], starts[e] + mt * bm, min(bm, lens[e] - mt * bm), False
    cols = [2 * p] + ([2 * p + 1] if 2 * p + 1 < ntn else [])
    return e, cols, starts[e] + F * bm, lens[e] - F * bm, True


def assign(total, grid, pool, rng):
    """Block -> item (static XCD ranges, optional shared pool in random order)."""
    q, r = total >> 3, total & 7
    n = [q + (x < r) for x in range(8)]
    t = [(nx + 15) >> 4 for nx in n]
    start = [x * q + min(x, r) for x in range(8)]
    items, takers = [], []
    for bid in range(grid):
        x, local = bid & 7, bid >> 3
        if not pool:
            if local < n[x]:
                items.append(start[x] + local)
        elif local < n[x] - t[x]:
            items.append(start[x] + local)
        elif local < n[x] + t[x]:
            takers.append(bid)
    rng.shuffle(takers)
    for i in range(len(takers)):
        base = 0
        for x in range(8):
            if i < base + t[x]:
                items.append(start[x] + n[x] - t[x] + i - base)
                break
            base += t[x]
    return items


def check(lens, ntn, pool, rng, bm=BM, half=HALF):
    starts = [sum(lens[:e]) for e in range(len(lens))]
    fp, hp = row_tiles(lens, bm, half)
    total = fp[-1] * ntn + hp[-1] * ((ntn + 1) >> 1)
    grid = total + rng.choice([0, 1, 7, 8, 9, total // 4 + 3])
    items = assign(total, grid, pool, rng)
    assert sorted(items) == list(range(total))
    covered = set()
    for L in items:
        e, cols, row0, rows, short = decode(L, fp, hp, ntn, lens, starts, bm)
        assert (1 <= rows <= half) if short else (half < rows <= bm)
        assert starts[e] <= row0 and row0 + rows <= starts[e] + lens[e]
        for c in cols:
            assert 0 <= c < ntn
            for rr in range(row0, row0 + rows):
                assert (c, rr) not in covered
                covered.add((c, rr))
    assert len(covered) == sum(lens) * ntn


@pytest.mark.parametrize("pool", [False, True])
def test_every_tile_once(pool):
    rng = random.Random(7)
    cases = [[0, 0, 1], [128, 129, 256, 257, 384, 385, 0, 1], [1] * 8, [255], [512, 640, 641, 1050, 1110, 2000],
             [0] * 5, [192, 193, 448, 449, 160]]
    for _ in range(16):
        E = rng.choice([3, 8, 33, 64])
        skew = rng.random() * 3
        cases.append([int(rng.random() ** skew * 700) for _ in range(E)] + [rng.choice([0, 300, 1025])])
    for lens in cases:
        for ntn in (1, 2, 3, 5, 16, 28):
            check(lens, ntn, pool, rng)


def test_fp32_tiles_never_short():
    rng = random.Random(3)
    for lens in ([1, 31, 32, 33, 64, 65, 0, 100], [5] * 9):
        for ntn in (1, 2, 3, 8, 9):
            check(lens, ntn, False, rng, bm=32, half=0)
