"""Host model of the multi-token kernel's LDS ring schedule (csrc/decode_multi.hip,
`begin_copies` and the tile loops): each wave's sequence of ring steps, K reads
and V reads, with the plain / general choice of every tile drawn at random per
wave (the kernel takes it per wave from its own scores). Checks, for the
pipelined row blocks (4 stages, copies 2 tiles ahead, tile m's V read after
tile m + 1 begins) and for the 16-row / head_dim-256 blocks (NS stages, copies
NS - 1 tiles ahead, each tile finished within its own step):

* every wave begins every tile once and in order, so all waves pass the same
  barriers;
* each tile is copied once, into stage tile % NS, by the begin LEAD tiles
  earlier (or before the loop);
* a tile's K and V are read only after its begin (its copies waited for, then
  the barrier);
* a stage is overwritten only after every wave has read the tile it held:
  each wave reads it before its own begin that issues the overwrite, and that
  begin's barrier orders every wave's reads before the copy;
* the outstanding copies a begin allows (LEAD - 1 later tiles) are exactly
  the tiles issued after the one begun.
"""
import random

import pytest


def wave_events(ntiles, pipe, plain):
    """Events of one wave: ("begin", j), ("K", j), ("V", j), in program order,
    following the kernel's loops; plain(m) is this wave's choice for tile m."""
    ev = []
    m = 0
    while m < ntiles:
        ev += [("begin", m), ("K", m)]
        if pipe:
            while m + 1 < ntiles and plain(m):
                # step: begin m + 1, read V of m, K of m + 1, update m
                ev += [("begin", m + 1), ("V", m), ("K", m + 1)]
                m += 1
        else:
            while plain(m):
                ev += [("V", m)]
                m += 1
                if m >= ntiles:
                    break
                ev += [("begin", m), ("K", m)]
            if m >= ntiles:
                break
        ev += [("V", m)]  # the general update of tile m
        m += 1
    return ev


def check_schedule(ntiles, NS, pipe, waves, seed):
    LEAD = NS - 2 if pipe else NS - 1
    rng = random.Random(seed)
    per_wave = []
    for w in range(waves):
        p = rng.random()
        choice = {m: rng.random() < p for m in range(ntiles)}
        per_wave.append(wave_events(ntiles, pipe, lambda m: choice[m]))
    for ev in per_wave:
        begins = [j for kind, j in ev if kind == "begin"]
        assert begins == list(range(ntiles)), "every tile begun once, in order"
        pos = {e: i for i, e in enumerate(ev)}
        for j in range(ntiles):
            assert pos[("K", j)] > pos[("begin", j)] and pos[("V", j)] > pos[("begin", j)]
        # copies: tiles 0..LEAD-1 before the loop, tile j + LEAD at begin(j)
        issued_at = {t: -1 for t in range(min(LEAD, ntiles))}
        for j in range(ntiles):
            if j + LEAD < ntiles:
                issued_at[j + LEAD] = j
        assert sorted(issued_at) == list(range(ntiles)), "each tile copied once"
        for t, j in issued_at.items():
            prev = t - NS  # the tile whose stage (t % NS) this copy overwrites
            if prev >= 0:
                assert j >= 0
                assert pos[("K", prev)] < pos[("begin", j)] and pos[("V", prev)] < pos[("begin", j)], \
                    f"stage of tile {prev} overwritten at begin {j} before its reads"
            if j >= 0:
                assert j < t, "copied ahead of its own begin"
        # at begin(j) the copies issued after tile j are tiles j+1 .. min(j+LEAD-1, ntiles-1)
        for j in range(ntiles):
            later = [t for t, at in issued_at.items() if t > j and at < j]
            assert len(later) == min(LEAD - 1, ntiles - 1 - j)


@pytest.mark.parametrize("pipe,NS", [(True, 4), (True, 3), (False, 3), (False, 2)])
@pytest.mark.parametrize("ntiles", [0, 1, 2, 3, 4, 5, 7, 16, 65])
def test_ring_schedule(pipe, NS, ntiles):
    for seed in range(40):
        check_schedule(ntiles, NS, pipe, 4, seed * 131 + ntiles)
