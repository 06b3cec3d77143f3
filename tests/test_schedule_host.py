"""Host-only checks of the stream-K work split used by the matrix-core arm
(mfma_gemm.h: sk_begin, sk_owner, the slot of a piece, the reduction's piece
walk, the dual GEMM's downward walk with in-kernel finishing), restated here
with the same integer formulas.

Workgroup g of G takes units [floor(g U / G), floor((g + 1) U / G)) of the
U = T * KU units; the workgroup that owns unit u is the largest g with
floor(g U / G) <= u; a piece of tile t held by workgroup g sits in slot
2 g + (t == first tile of g ? 0 : 1).
"""
import itertools

import pytest


def sk_begin(g, U, G):
    return g * U // G


def sk_owner(u, U, G):
    return ((u + 1) * G + U - 1) // U - 1


def slot(g, t, U, G, KU):
    return 2 * g + (0 if t == sk_begin(g, U, G) // KU else 1)


@pytest.mark.parametrize("T,KU", [(1, 1), (1, 7), (3, 5), (4, 4), (20, 272), (136, 80), (17, 3), (9, 64)])
def test_split_covers_every_unit_once_and_slots_are_unique(T, KU):
    U = T * KU
    for G in sorted({1, 2, 3, 5, 7, 16, 64, 255, 256, min(U, 256), U} & set(range(1, U + 1))):
        owner = {}
        for g in range(G):
            lo, hi = sk_begin(g, U, G), sk_begin(g + 1, U, G)
            assert hi > lo, "every workgroup gets at least one unit when G <= U"
            for u in range(lo, hi):
                assert u not in owner
                owner[u] = g
        assert sorted(owner) == list(range(U))
        for u in range(U):
            assert sk_owner(u, U, G) == owner[u]
        # pieces of each tile: contiguous workgroups g_lo..g_hi, distinct slots
        used = {}
        for t in range(T):
            g_lo, g_hi = sk_owner(t * KU, U, G), sk_owner(t * KU + KU - 1, U, G)
            assert {owner[u] for u in range(t * KU, (t + 1) * KU)} == set(range(g_lo, g_hi + 1))
            if g_lo == g_hi:
                continue  # whole tile in one workgroup: no slot
            for g in range(g_lo, g_hi + 1):
                s = slot(g, t, U, G, KU)
                assert 0 <= s < 2 * G
                assert s not in used, (t, g, used.get(s))
                used[s] = (t, g)


def test_whole_tiles_when_grid_equals_tiles():
    for T, KU in itertools.product([1, 5, 136], [1, 80]):
        U = T * KU
        for g in range(T):
            assert sk_begin(g, U, T) == g * KU
            assert sk_owner(g * KU + KU - 1, U, T) == g


def fix_walk(g, U, G, KU):
    """The dual GEMM's in-kernel finishing walk of workgroup g (its range in
    decreasing unit order, cut into pieces inside one tile), as actions:
    ("whole", t), ("piece", t, slot) or ("finish", t) -- the last only as the
    final action."""
    u_begin = sk_begin(g, U, G)
    n = sk_begin(g + 1, U, G) - u_begin
    acts, j = [], 0
    while j < n:
        top = u_begin + n - 1 - j
        t = top // KU
        lo = max(u_begin, t * KU)
        ku0, length = lo - t * KU, top - lo + 1
        j += length
        if ku0 == 0 and length == KU:
            acts.append(("whole", t))
            continue
        if ku0 + length == KU:
            assert j == n, "a split tile's top piece must be the workgroup's last"
            acts.append(("finish", t))
            break
        acts.append(("piece", t, slot(g, t, U, G, KU)))
    return acts


@pytest.mark.parametrize("T,KU", [(1, 7), (3, 5), (4, 4), (136, 80), (34, 80), (17, 3), (9, 64), (272, 80)])
def test_in_kernel_finishing_walk(T, KU):
    """Every split tile has exactly one finisher, the sharer that holds its top
    unit; the other sharers each leave one piece in their slot; the finisher
    reads exactly those slots and waits only for lower-numbered workgroups;
    every unit is covered once."""
    U = T * KU
    for G in sorted({1, 2, 3, 7, 64, 255, 256, min(U, 256)} & set(range(1, U + 1))):
        whole, pieces, finisher = {}, {}, {}
        for g in range(G):
            acts = fix_walk(g, U, G, KU)
            assert sum(a[0] == "finish" for a in acts) <= 1
            assert {a[2] for a in acts if a[0] == "piece"} <= {2 * g, 2 * g + 1}
            for a in acts:
                if a[0] == "whole":
                    assert a[1] not in whole
                    whole[a[1]] = g
                elif a[0] == "piece":
                    pieces.setdefault(a[1], {})[g] = a[2]
                else:
                    assert a[1] not in finisher
                    finisher[a[1]] = g
        for t in range(T):
            g_lo, g_hi = sk_owner(t * KU, U, G), sk_owner(t * KU + KU - 1, U, G)
            if g_lo == g_hi:
                assert whole.get(t) == g_lo and t not in finisher and t not in pieces
                continue
            assert t not in whole
            assert finisher[t] == g_hi
            # what the finisher reads: slot 2 gg + (t is gg's first tile ? 0 : 1), gg = g_hi - 1 .. g_lo
            reads = {gg: slot(gg, t, U, G, KU) for gg in range(g_hi - 1, g_lo - 1, -1)}
            assert pieces[t] == reads
            assert all(gg < g_hi for gg in reads)
        assert set(whole) | set(finisher) == set(range(T))
