"""Host model of the stream-K work split of the bf16 GEMM (the same integer formulas
the product and fixup kernels evaluate per workgroup and per tile), checked for the
properties the kernels rely on: the whole rounds' tiles are each taken by exactly one
workgroup, in the tile kernel's XCD order; every (tile, k-stage) unit of the
remaining tiles is covered by exactly one run; a run has at most two partial
segments (its first and its last), so two workspace slots per run suffice; the slots
the fixup reads for a split tile are distinct and are the ones its runs wrote; and
the split is used only when the last round of tiles is at most half full."""
import itertools

import pytest

GRID, BK = 256, 32


MIN_STAGES, MAX_TILES = 48, 1023


def sk_applies(tiles, K):
    return (K >= MIN_STAGES * BK and tiles > 0 and tiles % GRID != 0 and tiles % GRID <= GRID // 2
            and tiles <= MAX_TILES and tiles * ((K + BK - 1) // BK) < (1 << 30))


def whole_tiles(T):
    """Workgroup b's whole tiles: (b % 8) * D / 8 + b / 8 + 32 i, D = 256 * floor(T / 256)."""
    rounds = T // GRID
    D = rounds * GRID
    return D, [[(b % 8) * (D // 8) + b // 8 + i * (GRID // 8) for i in range(rounds)] for b in range(GRID)]


def runs(T, nk):
    """The runs over the remainder's units (tiles counted from D)."""
    R = T - T // GRID * GRID
    U = R * nk
    per = (U + GRID - 1) // GRID
    return U, per, [(min(U, v * per), min(U, min(U, v * per) + per)) for v in range(GRID)]


def written_slots(T, nk):
    """(tile, run) -> slot written by the product kernel for each split segment."""
    U, per, rr = runs(T, nk)
    out = {}
    for v, (g0, g1) in enumerate(rr):
        gs = g0
        segs = 0
        while gs < g1:
            ti = gs // nk
            kb, ke = gs - ti * nk, min(nk, g1 - ti * nk)
            if kb != 0 or ke != nk:
                segs += 1
                out[(ti, v)] = 2 * v + (0 if ti == v * per // nk else 1)
            gs = ti * nk + ke
        assert segs <= 2
    return out


@pytest.mark.parametrize("T", [1, 2, 8, 64, 120, 264, 384, 576, 864, 1152, 3456])
def test_whole_tiles(T):
    D, lists = whole_tiles(T)
    taken = sorted(t for l in lists for t in l)
    assert taken == list(range(D))
    # an XCD's workgroups take consecutive tiles in each round
    for b in range(GRID):
        for i, t in enumerate(lists[b]):
            assert t == lists[b % 8][i] + b // 8


@pytest.mark.parametrize("T,nk", list(itertools.product([1, 2, 8, 64, 120, 264, 384, 576, 864, 1152, 3456],
                                                        [1, 3, 16, 64, 384])))
def test_partition(T, nk):
    U, per, rr = runs(T, nk)
    T = T - T // GRID * GRID  # the remainder's tiles, counted from D
    cover = [0] * U
    for g0, g1 in rr:
        assert 0 <= g0 <= g1 <= U
        for u in range(g0, g1):
            cover[u] += 1
    assert all(c == 1 for c in cover)
    w = written_slots(T, nk)
    assert len(set(w.values())) == len(w) and all(0 <= s < 2 * GRID for s in w.values())
    for ti in range(T):
        ua = ti * nk
        vf, vl = ua // per, (ua + nk - 1) // per
        if vf == vl:
            assert all(t != ti for (t, _) in w)  # finished by its only run, nothing written
            continue
        read = [2 * u + (0 if ti == u * per // nk else 1) for u in range(vf, vl + 1)]
        assert read == [w[(ti, u)] for u in range(vf, vl + 1)]


def test_rule():
    assert not sk_applies(256, 12288) and not sk_applies(512, 6144)     # whole rounds
    assert sk_applies(64, 12288) and sk_applies(264, 12288)             # last round <= half full
    assert sk_applies(384, 12288) and sk_applies(576, 18432) and sk_applies(864, 4096)
    assert not sk_applies(192, 12288)                                    # 3/4 full: tile kernel
    assert not sk_applies(1152, 2048) and not sk_applies(2592, 4096)    # four rounds or more: tile kernel
    assert not sk_applies(3456, 4096)
    assert not sk_applies(64, 1504) and sk_applies(64, 1536)            # at least 48 k-stages
    assert not sk_applies(5000, 64) and not sk_applies(64, 0)
