"""CPU check of the lane schedule of the wave-level combine scan that gives
the time segments their carry-ins (segment_carry_kernel): four doubling
steps inside each 16-lane row (each lane combines the pair of the lane 1, 2,
4, 8 below it in its row, lanes without one take the identity), then rows 1
and 3 combine lane 15 of the row before them, then rows 2 and 3 combine
lane 31.  Simulated exactly in rationals over 64 lanes, the result must be
the sequential prefix of the combine operator of "Mamba CUDA 实现解析"
eq. (10) for every lane, for every number of active lanes (inactive lanes
hold the identity)."""
import random
from fractions import Fraction

import pytest


def combine(left, right):
    """(a_l, v_l) (+) (a_r, v_r) = (a_r a_l, a_r v_l + v_r): left is earlier."""
    (al, vl), (ar, vr) = left, right
    return (ar * al, ar * vl + vr)


IDENT = (Fraction(1), Fraction(0))


def dpp_step(vals, src_of, rows_enabled):
    """One scan_step: lane i combines the pair of lane src_of(i) (None: no
    source) on its left, if its 16-lane row is enabled; else the identity."""
    out = []
    for i, x in enumerate(vals):
        j = src_of(i)
        if (i // 16) not in rows_enabled or j is None:
            prev = IDENT
        else:
            prev = vals[j]
        out.append(combine(prev, x))
    return out


def wave_scan(vals, rpp=4):
    """rpp: 16-lane rows per sequence (1, 2 or 4), 4 // rpp sequences side by side."""
    for off in (1, 2, 4, 8):                  # row_shr:off, all rows
        vals = dpp_step(vals, lambda i, o=off: i - o if (i % 16) >= o else None, {0, 1, 2, 3})
    if rpp >= 2:  # row_bcast:15 -> rows 1 and 3 read lane 15 of the row before
        vals = dpp_step(vals, lambda i: (i // 16) * 16 - 1, {1, 3})
    if rpp == 4:  # row_bcast:31 -> rows 2 and 3 read lane 31
        vals = dpp_step(vals, lambda i: 31, {2, 3})
    return vals


@pytest.mark.parametrize("active", [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64])
def test_wave_scan_schedule_is_the_sequential_prefix(active):
    rng = random.Random(active)
    items = [(Fraction(rng.randint(1, 9), rng.randint(1, 9)),
              Fraction(rng.randint(-9, 9), rng.randint(1, 9))) for _ in range(active)]
    lanes = items + [IDENT] * (64 - active)
    got = wave_scan(lanes)
    acc = IDENT
    for i in range(active):
        acc = combine(acc, items[i])
        assert got[i] == acc, i


def test_carry_from_initial_state_reversed_order():
    """The adjoint direction: lane j holds the aggregate of segment n-1-j, so
    the lane scan composes the segments from the right; the carry of a
    segment is the composition applied to the initial value."""
    rng = random.Random(7)
    n = 20
    aggs = [(Fraction(rng.randint(1, 5), 7), Fraction(rng.randint(-5, 5), 3)) for _ in range(n)]
    init = Fraction(3, 2)
    lanes = [aggs[n - 1 - j] for j in range(n)] + [IDENT] * (64 - n)
    got = wave_scan(lanes)
    for s in range(n):          # carry entering segment s - 1 from the right ...
        j = n - 1 - s
        lam = init
        for t in range(n - 1, s - 1, -1):   # ... = aggregates n-1 .. s applied in turn
            a, v = aggs[t]
            lam = a * lam + v
        a, v = got[j]
        assert a * init + v == lam


@pytest.mark.parametrize("rpp,active", [(1, 1), (1, 5), (1, 15), (1, 16),
                                         (2, 1), (2, 16), (2, 17), (2, 31), (2, 32)])
def test_side_by_side_sequences(rpp, active):
    """Shorter sequences (at most 16 or 32 segments) packed 4 or 2 to a wave:
    each sequence's lanes get its own sequential prefix, untouched by its
    neighbours."""
    width = 16 * rpp
    rng = random.Random(100 * rpp + active)
    seqs = [[(Fraction(rng.randint(1, 9), rng.randint(1, 9)),
              Fraction(rng.randint(-9, 9), rng.randint(1, 9))) for _ in range(active)]
            for _ in range(4 // rpp)]
    lanes = []
    for sq in seqs:
        lanes += sq + [IDENT] * (width - active)
    got = wave_scan(lanes, rpp)
    for j, sq in enumerate(seqs):
        acc = IDENT
        for i in range(active):
            acc = combine(acc, sq[i])
            assert got[j * width + i] == acc, (j, i)
