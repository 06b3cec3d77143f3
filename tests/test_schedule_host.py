"""Host-only checks of the stream-K work split used by the matrix-core arm
(mfma_gemm.h: sk_begin, sk_owner, the slot of a piece, the reduction's piece
walk), restated here with the same integer formulas.

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
