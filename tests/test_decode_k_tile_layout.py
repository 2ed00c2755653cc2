"""Host model of the K tile of the matrix-core decode kernel (head_dim 128,
16-bit K): each lane loads whole-row segments like V (lane (r, c) of a
wave64, lane = 16 r + c: row 4 j + r of the 16-key tile, 16-byte segment c,
for load j = 0..3), writes them to a per-wave LDS tile with segment s of row
k at slot s ^ k, and reads back the MFMA A operand of k-step j (MFMA row c
holds key (c % 4) * 4 + c / 4; lane (r, c) needs that key's dims
32 j + 8 r .. + 8, i.e. its segment 4 j + r). The index rules are restated
from decode_split_mfma.hip. Checks: every slot of the tile is written once,
every lane reads exactly its operand segment, and the 16 lanes of one r
touch 16 different 16-byte slots in every write and every read."""

D = 128
TR = 16            # keys per tile
NSL = D // 8       # 16-byte segments (slots) per row
NJ = D // 32       # loads per tile = MFMA k-steps


def key_of_lane(c):
    return (c & 3) * 4 + (c >> 2)


def write_tile():
    """slot contents after the four loads: tile[row][slot] = (row, segment)."""
    tile = [[None] * NSL for _ in range(TR)]
    for j in range(NJ):
        for lane in range(64):
            r, c = lane // 16, lane % 16
            row, seg = 4 * j + r, c                  # what the lane loaded
            slot = c ^ (4 * j + r)
            assert tile[row][slot] is None, "slot written twice"
            tile[row][slot] = (row, seg)
    return tile


def test_every_slot_written_once():
    tile = write_tile()
    assert all(x is not None for row in tile for x in row)
    # each row holds each of its segments once
    for row in range(TR):
        assert sorted(seg for (rw, seg) in tile[row]) == list(range(NSL))
        assert all(rw == row for (rw, seg) in tile[row])


def test_operand_reads_get_the_mfma_layout():
    tile = write_tile()
    for j in range(NJ):
        for lane in range(64):
            r, c = lane // 16, lane % 16
            k = key_of_lane(c)
            got = tile[k][(4 * j + r) ^ k]
            assert got == (k, 4 * j + r)             # row k, dims 32 j + 8 r .. + 8


def test_key_mapping_matches_the_score_layout():
    # MFMA result register i of lane (r, c) is output row 4 r + i; with row m
    # holding key (m % 4) * 4 + m / 4 that is key 4 i + r: the keys whose V
    # rows lane (r, c) loads (rows 4 i + r).
    for r in range(4):
        for i in range(4):
            assert key_of_lane(4 * r + i) == 4 * i + r
    assert sorted(key_of_lane(c) for c in range(16)) == list(range(16))


def xor_slot(seg, row):
    return seg ^ row


def plain_slot(seg, row):
    return seg


def slot_spread(slot):
    """Smallest number of distinct slots the 16 lanes of one r touch, over
    every write and every operand read of the tile."""
    worst = 16
    for j in range(NJ):
        for r in range(4):
            writes = {slot(c, 4 * j + r) for c in range(16)}                 # row 4 j + r, segment c
            reads = {slot(4 * j + r, key_of_lane(c)) for c in range(16)}     # row key, segment 4 j + r
            worst = min(worst, len(writes), len(reads))
    return worst


def test_sixteen_lanes_hit_sixteen_slots():
    assert slot_spread(xor_slot) == 16


def test_without_the_xor_reads_would_share_one_slot():
    # planted mistake: segment s of every row at slot s puts the 16 lanes of
    # an operand read (one segment of 16 rows) on one slot
    assert slot_spread(plain_slot) == 1
