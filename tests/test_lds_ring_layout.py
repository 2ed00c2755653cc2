"""Host model of the multi-token LDS-ring layout (head_dim 64, 128, 256): the
1 KiB global->LDS copies, the K operand reads and the 16-bit transposing V^T
reads, with the slot permutation of decode_multi.hip restated here. Checks
that every lane receives exactly the K and V^T operand elements of the MFMA
layout, that every LDS element is written once, and the bank spreads the
permutation is designed for (32 lanes of a transposing read on 32 different
8-byte units of the 64 four-byte banks; 16 lanes of a K read on 16 different
16-byte units). The transposing read follows the lane rule measured on the
GPU: within each 16-lane group, lane i receives element i % 4 of the 8-byte
rows addressed by lanes (i % 16) / 4 + 4 j, j = 0..3."""
import pytest

KT = 32


def swz(D, k):
    if D == 64:
        return (((k >> 1) & 3) << 1) | ((k >> 3) & 1)
    return ((k & 7) << 1) | (((k >> 2) ^ (k >> 3)) & 1)


def val(key, dim):
    return key * 1000 + dim


def build_stage(D):
    """LDS contents of one stage after the four waves' copies (element index -> (key, dim))."""
    RB, NSEG, KPC = 2 * D, D // 8, 512 // D
    lds = [None] * (KT * D)
    for w in range(4):
        for j in range(D // 64):
            base = (8 * w + KPC * j) * D
            for i in range(64):
                krow = KPC * j + i // NSEG
                key = 8 * w + krow
                c = (i % NSEG) ^ swz(D, key)       # global segment this lane loads
                loff = krow * RB + 16 * c           # its byte offset from key 8w's row
                assert loff // RB == krow and 0 <= c < NSEG
                for t in range(8):
                    e = base + i * 8 + t
                    assert lds[e] is None
                    lds[e] = val(key, c * 8 + t)
    assert all(x is not None for x in lds)
    return lds


@pytest.mark.parametrize("D", [64, 128, 256])
def test_k_operand_reads(D):
    lds = build_stage(D)
    for lane in range(64):
        col, q4 = lane & 15, lane >> 4
        for kb in range(2):
            for ks in range(D // 32):
                e0 = (kb * 16 + col) * D + ((4 * ks + q4) ^ swz(D, col)) * 8
                assert lds[e0:e0 + 8] == [val(kb * 16 + col, 32 * ks + 8 * q4 + t) for t in range(8)]
    for q4 in range(4):
        for ks in range(D // 32):
            units = {((col * D + ((4 * ks + q4) ^ swz(D, col)) * 8) * 2 % 256) // 16 for col in range(16)}
            assert len(units) == 16


@pytest.mark.parametrize("D", [64, 128, 256])
def test_transposing_v_reads(D):
    lds = build_stage(D)
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
