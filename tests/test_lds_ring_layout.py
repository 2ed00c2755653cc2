"""Host model of the multi-token LDS-ring layout (head_dim 64, 128, 256): the
1 KiB global->LDS copies of K and V, the K operand reads and the 16-bit
transposing V^T reads, with the copy addressing and the layouts of
decode_multi.hip restated here. Checks that every lane receives exactly the K
and V^T operand elements of the MFMA layout, that every LDS element is
written once, that each copy reads whole 128-byte lines of a wave's own 8
keys (one page), and the bank spreads the layouts are designed for (the 16
lanes of a K read on two 128-byte runs in opposite halves of the 64
four-byte banks; 32 lanes of a transposing V read on 32 different 8-byte
units). The transposing read follows the lane rule measured on the GPU:
within each 16-lane group, lane i receives element i % 4 of the 8-byte rows
addressed by lanes (i % 16) / 4 + 4 j, j = 0..3."""
import pytest

KT = 32


def swz(D, k):
    if D == 64:
        return (((k >> 1) & 3) << 1) | ((k >> 3) & 1)
    return ((k & 7) << 1) | (((k >> 2) ^ (k >> 3)) & 1)


def val(key, dim):
    return key * 1000 + dim


def build_k_stage(D):
    """K stage after the four waves' copies: element -> (key, dim)."""
    RB, NSEG = 2 * D, D // 8
    lds = [None] * (KT * D)
    for w in range(4):
        for j in range(D // 64):
            lines = set()
            for i in range(64):
                seg = (8 * j + i // 8) ^ (w & 1)
                koff = (i % 8) * RB + 16 * seg              # bytes from the row of key 8w
                key = 8 * w + koff // RB
                assert 0 <= seg < NSEG and key == 8 * w + i % 8
                lines.add((key, (koff % RB) // 128))
                for t in range(8):
                    e = 8 * w * D + 512 * j + 8 * i + t
                    assert lds[e] is None
                    lds[e] = val(key, seg * 8 + t)
            # whole 128-byte lines: 8 rows x 128 bytes per copy
            assert len(lines) == 8
    assert all(x is not None for x in lds)
    return lds


def build_v_stage(D):
    """V stage after the four waves' copies: element -> (key, dim)."""
    RB, NSEG, KPC = 2 * D, D // 8, 512 // D
    lds = [None] * (KT * D)
    for w in range(4):
        for j in range(D // 64):
            base = (8 * w + KPC * j) * D
            for i in range(64):
                krow = KPC * j + i // NSEG
                c = (i % NSEG) ^ swz(D, 8 * w + krow)
                key = 8 * w + krow
                assert krow < 8
                for t in range(8):
                    e = base + i * 8 + t
                    assert lds[e] is None
                    lds[e] = val(key, c * 8 + t)
    assert all(x is not None for x in lds)
    return lds


def k_read(D, lane, kb, ks):
    NSEG = D // 8
    col, q4 = lane & 15, lane >> 4
    g = col >> 3
    return g * (NSEG * 64) + (q4 ^ g) * 64 + (col & 7) * 8 + kb * (2 * NSEG * 64) + ks * 256


@pytest.mark.parametrize("D", [64, 128, 256])
def test_k_operand_reads(D):
    lds = build_k_stage(D)
    for lane in range(64):
        col, q4 = lane & 15, lane >> 4
        for kb in range(2):
            for ks in range(D // 32):
                e0 = k_read(D, lane, kb, ks)
                assert lds[e0:e0 + 8] == [val(kb * 16 + col, 32 * ks + 8 * q4 + t) for t in range(8)]
    # the 16 lanes of one read: two 128-byte runs in opposite bank halves
    for kb in range(2):
        for ks in range(D // 32):
            for q4 in range(4):
                byte = [k_read(D, q4 * 16 + col, kb, ks) * 2 for col in range(16)]
                for g in range(2):
                    run = byte[8 * g:8 * g + 8]
                    assert run == list(range(run[0], run[0] + 128, 16))
                assert {b % 256 // 128 for b in byte[:8]} != {b % 256 // 128 for b in byte[8:]}


@pytest.mark.parametrize("D", [64, 128, 256])
def test_k_rows_of_16_row_blocks(D):
    """The 16-row blocks keep K in rows like V (whole-row copies): operand
    read of key 16 kb + col at slot (4 ks + q4) ^ swz(col)."""
    lds = build_v_stage(D)
    for lane in range(64):
        col, q4 = lane & 15, lane >> 4
        for kb in range(2):
            for ks in range(D // 32):
                e0 = col * D + kb * 16 * D + ((4 * ks + q4) ^ swz(D, col)) * 8
                assert lds[e0:e0 + 8] == [val(kb * 16 + col, 32 * ks + 8 * q4 + t) for t in range(8)]


@pytest.mark.parametrize("D", [64, 128, 256])
def test_transposing_v_reads(D):
    lds = build_v_stage(D)
    for nb in range(D // 16):
        for r in range(2):
            addrs = []
            for lane in range(64):
                col, q4 = lane & 15, lane >> 4
                vkey = 4 * q4 + (col >> 2)
                addrs.append(vkey * D + (((2 * nb + ((col & 3) >> 1)) ^ swz(D, vkey)) * 8) + (col & 1) * 4
                             + r * 16 * D)
            for lane in range(64):
                col, q4 = lane & 15, lane >> 4
                src = [addrs[(lane & ~15) + (lane % 16) // 4 + 4 * j] + lane % 4 for j in range(4)]
                assert [lds[e] for e in src] == [val(16 * r + 4 * q4 + j, 16 * nb + col) for j in range(4)]
            for h in range(2):
                assert len({(addrs[h * 32 + t] * 2 % 256) // 8 for t in range(32)}) == 32


def test_a_plain_permutation_would_conflict():
    """The property is not vacuous: without the row-dependent part (swz = 0)
    the 32 lanes of a transposing read share 8-byte units."""
    D = 128
    addrs = []
    for lane in range(32):
        col, q4 = lane & 15, lane >> 4
        vkey = 4 * q4 + (col >> 2)
        addrs.append(vkey * D + ((2 * 0 + ((col & 3) >> 1)) * 8) + (col & 1) * 4)
    assert len({(a * 2 % 256) // 8 for a in addrs}) < 32


def test_unswapped_second_block_would_conflict():
    """The property is not vacuous: without the swap in odd blocks the two
    128-byte runs of a K read share one half of the banks."""
    D = 128
    NSEG = D // 8
    byte = [((col >> 3) * (NSEG * 64) + 0 * 64 + (col & 7) * 8) * 2 for col in range(16)]
    assert {b % 256 // 128 for b in byte[:8]} == {b % 256 // 128 for b in byte[8:]}
