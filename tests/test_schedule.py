"""The causal forward's persistent schedule, modelled on the CPU.

Under the causal mask ``fa_fwd_kernel.hip`` launches one workgroup per
resident slot (rounded up to a multiple of 8) and deals the work items --
single q blocks of one (batch, query head) row group -- to them: the row
groups are cut into 8 contiguous ranges, one per XCD; an XCD walks its range
in phases of C row groups, and a phase's items, ordered heaviest first
(block nQ-1 of each of its row groups, then nQ-2, ...), are dealt in rounds
whose direction alternates (with several phases, to a permuted slot order
that gives a row group consecutive slots).  This model repeats that index arithmetic and
checks that every item is dealt exactly once, that every workgroup is on
the XCD of its row groups, that a phase holds few row groups, and that the
work per workgroup is balanced on the benchmark shapes.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

XCDS = 8


def grid_for(items, slots):
    want = min(items, slots)
    return (want + XCDS - 1) // XCDS * XCDS


def phase_rows(rows, nq, grid):
    """The host's C0 = 2 gx / gcd(nQ, 2 gx)."""
    gx2 = 2 * (grid // XCDS if rows >= XCDS else grid)
    return gx2 // math.gcd(nq, gx2)


def schedule(rows, nq, grid):
    """Items (row group, q block) of each workgroup, in the order it runs them."""
    c0 = phase_rows(rows, nq, grid)
    out = []
    for blk in range(grid):
        gx, s, rg0, nrg = grid, blk, 0, rows
        if rows >= XCDS:
            x = blk % XCDS
            per, extra = divmod(rows, XCDS)
            rg0 = x * per + min(x, extra)
            nrg = per + (1 if x < extra else 0)
            gx //= XCDS
            s //= XCDS
        c = c0 if nrg % c0 == 0 else nrg
        if c < nrg and gx % c == 0:  # several phases: a row group's slots made consecutive
            m = gx // c
            s = (s % m) * c + s // m
        mine = []
        for p0 in range(0, nrg, c):
            n = c * nq
            r = 0
            while True:
                idx = r * gx + (gx - 1 - s if r & 1 else s)
                if idx >= n:
                    break
                assert idx < 2 ** 31
                mine.append((rg0 + p0 + idx % c, nq - 1 - idx // c))
                r += 1
        out.append(mine)
    return out


@pytest.mark.parametrize("rows", [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 64, 100, 256])
@pytest.mark.parametrize("nq", [1, 2, 3, 5, 8, 33])
@pytest.mark.parametrize("slots", [8, 24, 256, 512, 768])
def test_every_item_dealt_once(rows, nq, slots):
    grid = grid_for(rows * nq, slots)
    got = [it for wg in schedule(rows, nq, grid) for it in wg]
    assert len(got) == rows * nq
    assert set(got) == {(rg, qb) for rg in range(rows) for qb in range(nq)}


@pytest.mark.parametrize("rows,nq,slots", [(256, 8, 768), (256, 32, 512), (64, 32, 256), (32, 64, 256),
                                           (17, 5, 768)])
def test_row_groups_stay_on_their_xcd(rows, nq, slots):
    grid = grid_for(rows * nq, slots)
    per, extra = divmod(rows, XCDS)
    home = {}
    for x in range(XCDS):
        first = x * per + min(x, extra)
        for rg in range(first, first + per + (1 if x < extra else 0)):
            home[rg] = x
    for blk, items in enumerate(schedule(rows, nq, grid)):
        for rg, _ in items:
            assert home[rg] == blk % XCDS


def test_heaviest_first_within_a_workgroup():
    for items in schedule(256, 8, 768):
        assert items and items[0][1] == max(qb for _, qb in items)


@pytest.mark.parametrize("rows,nq,slots,c", [(256, 32, 512, 4), (256, 16, 256, 4), (64, 32, 256, 2), (32, 64, 256, 1),
                                             (256, 8, 512, 16)])
def test_phases_hold_few_row_groups(rows, nq, slots, c):
    """Where a phase divides an XCD's range, the workgroups of an XCD work
    on at most 2 C row groups at a time (the items of one round lie in at
    most two consecutive phases) -- the K/V that must stay in its L2."""
    grid = grid_for(rows * nq, slots)
    assert phase_rows(rows, nq, grid) == c
    sched = schedule(rows, nq, grid)
    for x in range(XCDS):
        wgs = [sched[b] for b in range(x, grid, XCDS)]
        for r in range(max(len(w) for w in wgs)):
            live = {w[r][0] for w in wgs if r < len(w)}
            assert len(live) <= 2 * c


# Benchmark shapes: (rows = B*H, Lq, Lk, q rows per workgroup, resident slots)
SHAPES = {
    "B=8 H=32 L=1024 D=64 causal (W=4, 3 workgroups/CU)": (256, 1024, 1024, 128, 768),
    "B=8 H=32 L=4096 D=128 causal (W=8)": (256, 4096, 4096, 256, 256),
    "B=8 H=32 L=2048 D=128 causal (W=4, 2 workgroups/CU)": (256, 2048, 2048, 128, 512),
    "GQA B=2 H=32 L=8192 D=128 causal (W=8)": (64, 8192, 8192, 256, 256),
    "B=1 H=32 L=16384 D=128 causal (W=8)": (32, 16384, 16384, 256, 256),
    "prefill B=8 H=32 1024 queries after 3072 keys (W=8)": (256, 1024, 4096, 256, 256),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_balanced_on_benchmark_shapes(name):
    """Keys seen per workgroup (the causal cost of an item is the keys its
    q block sees): the busiest workgroup does at most 10 % more than the
    mean.  (Units of two blocks (nQ-1-i, i), equal in cost, would leave the
    D = 64 shape, 1024 pairs on 768 workgroups, at twice the work on a third
    of them.)"""
    rows, lq, lk, bm, slots = SHAPES[name]
    past = lk - lq
    nq = (lq + bm - 1) // bm
    grid = grid_for(rows * nq, slots)

    def cost(qb):
        return min(lk, past + min((qb + 1) * bm, lq))

    load = np.array([sum(cost(qb) for _, qb in wg) for wg in schedule(rows, nq, grid)], dtype=np.float64)
    assert load.max() <= 1.10 * load.mean(), (load.max(), load.mean())
