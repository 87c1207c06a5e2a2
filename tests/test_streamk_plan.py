"""Host-side check of the K-split tail's indexing (the integer arithmetic of
plan_stream_k, sk_item and sk_fixup_kernel in csrc/gemm_bf16.hip, restated):
with Tt tail tiles of KS K steps, q = min(⌊256/Tt⌋, KS) pieces of
L = ⌈KS/q⌉ steps per tile (q then recounted as the non-empty ones), item
c = j·Tt + u covers steps [j·L, min((j+1)·L, KS)) of tile u and writes slot
c; together the items cover every (tile, step) exactly once, there are at
most 256 of them, pieces of one index j have the same K range in every
tile, and the fix-up of tile u reads slots j·Tt + u for j < q, in K order.
No GPU."""

import itertools

import pytest

P = 256  # compute units


def plan(Tt, KS):
    q = min(P // Tt, KS)
    if q < 2:
        return None
    L = -(-KS // q)
    q = -(-KS // L)
    return q, L


@pytest.mark.parametrize("Tt,KS", list(itertools.product([1, 2, 16, 31, 100, 128, 129, 144, 255],
                                                       [2, 3, 4, 10, 24, 48, 200, 400])))
def test_tail_pieces_cover_each_tile_once_in_k_order(Tt, KS):
    pl = plan(Tt, KS)
    if pl is None:
        assert P // Tt < 2 or KS < 2
        return
    q, L = pl
    assert Tt * q <= P
    written = {}
    for c in range(Tt * q):
        j, u = divmod(c, Tt)
        kb = j * L
        assert j < q and kb < KS  # no empty item
        written[c] = (u, kb, min(kb + L, KS))
    cover = set()
    for u, kb, ke in written.values():
        for k in range(kb, ke):
            assert (u, k) not in cover
            cover.add((u, k))
    assert len(cover) == Tt * KS
    for u in range(Tt):
        pieces = [written[j * Tt + u] for j in range(q)]
        assert pieces[0][1] == 0 and pieces[-1][2] == KS
        for a, b in zip(pieces, pieces[1:]):
            assert a[2] == b[1]
    # same K range for every tile at each piece index
    for j in range(q):
        assert len({written[j * Tt + u][1:] for u in range(Tt)}) == 1
