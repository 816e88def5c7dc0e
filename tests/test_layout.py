"""CPU model of the swizzled row tiles the backward kernels stage in LDS.

A 32 x 128 bf16 tile is stored with 256-byte rows; the 16-byte chunk c of row r
sits at chunk position c ^ row_swz(r). The kernels fill a tile with 1 KB direct
copies and read it two ways: 16-byte reads that give MFMA A fragments (lane ->
row, 8 consecutive columns) and pairs of transposing 8-byte reads that give B
fragments whose k index runs over rows (lane -> column, 8 rows). This test
re-derives every lane's bytes from the address formulas and checks that each
fragment holds the elements the 32x32x16 bf16 MFMA expects, and that the 16
lanes of each transposing read cover 16 distinct 4-byte banks mod 64 per 4-lane
row group. The formulas mirror exact_shared_prefix_amd/csrc/frag.h. Pure
Python, no GPU.
"""
import numpy as np


def row_swz(r):
    return 4 * (r & 3) + ((r >> 2) & 3)


def row_a_base(lane):
    r, hl = lane & 31, lane >> 5
    return 256 * r + 16 * (row_swz(r) ^ hl)


def row_b_base(lane):
    g, L = lane >> 4, lane & 15
    a, j = L & 3, L >> 2
    hl, x = g >> 1, g & 1
    return 1024 * hl + 320 * j + 8 * (a & 1) + 16 * ((2 * x + (a >> 1)) ^ hl)


def element_at(byte):
    """(row, column) of the bf16 element stored at a byte offset of the tile."""
    r, w = divmod(byte, 256)
    c = (w // 16) ^ row_swz(r)
    return r, 8 * c + (w % 16) // 2


def copy_layout():
    """Tile bytes after the 8 direct copies: copy m, lane l fetches row
    4m + l/16, chunk (l % 16) ^ row_swz(row) and lands at byte 1024 m + 16 l."""
    where = {}
    for m in range(8):
        for lane in range(64):
            r = 4 * m + lane // 16
            c = (lane % 16) ^ row_swz(r)
            dst = 1024 * m + 16 * lane
            for e in range(8):
                where[dst + 2 * e] = (r, 8 * c + e)
    return where


def test_copies_place_every_element_where_the_swizzle_says():
    where = copy_layout()
    assert len(where) == 32 * 128
    for byte, rc in where.items():
        assert element_at(byte) == rc
    assert sorted(where.values()) == [(r, c) for r in range(32) for c in range(128)]


def test_a_fragments():
    # 32x32x16 A operand: lane l holds row l % 32, k = 8 (l / 32) + 0..7 of
    # the 16-column step kk
    for kk in range(8):
        for lane in range(64):
            base = row_a_base(lane) ^ (32 * kk)
            assert base % 16 == 0
            got = [element_at(base + 2 * e) for e in range(8)]
            want = [(lane % 32, 16 * kk + 8 * (lane // 32) + e) for e in range(8)]
            assert got == want, (kk, lane)


def tr16_b64(addrs):
    """The transposing 8-byte read: lane i of each 16-lane group gets, in slot
    j, element i % 4 of the 4 elements at the address of lane i / 4 + 4 j of
    its group."""
    out = []
    for lane in range(64):
        g, i = divmod(lane, 16)
        slots = []
        for j in range(4):
            src = 16 * g + i // 4 + 4 * j
            r, c = element_at(addrs[src])
            slots.append((r, c + i % 4))
        out.append(slots)
    return out


def test_b_fragments_from_transposing_reads():
    # B operand with k over rows: lane l holds column 32 dt + l % 32 and, in
    # slot 4 h + j, row 16 ks + 8 h + 4 (l / 32) + j (the accumulator row order
    # of the P / dS fragments it is paired with)
    for ks in range(2):
        for dt in range(4):
            halves = []
            for h in range(2):
                addrs = [4096 * ks + 2048 * h + (row_b_base(lane) ^ (64 * dt + 32 * h)) for lane in range(64)]
                assert all(a % 8 == 0 for a in addrs)
                halves.append(tr16_b64(addrs))
            for lane in range(64):
                got = halves[0][lane] + halves[1][lane]
                want = [(16 * ks + 8 * (e // 4) + 4 * (lane // 32) + e % 4, 32 * dt + lane % 32) for e in range(8)]
                assert got == want, (ks, dt, lane)


def test_reads_spread_over_banks():
    # every 16-lane quarter of an A-fragment read touches 64 distinct 4-byte
    # banks (16 lanes x 16 bytes), and every 32-lane half of a transposing
    # read touches 64 distinct banks (32 lanes x 8 bytes)
    for kk in range(8):
        for q in range(4):
            banks = set()
            for lane in range(16 * q, 16 * q + 16):
                b = row_a_base(lane) ^ (32 * kk)
                banks.update(((b // 4) + t) % 64 for t in range(4))
            assert len(banks) == 64, (kk, q)
    for dt in range(4):
        for h in range(2):
            for half in range(2):
                banks = set()
                for lane in range(32 * half, 32 * half + 32):
                    b = 2048 * h + (row_b_base(lane) ^ (64 * dt + 32 * h))
                    banks.update(((b // 4) + t) % 64 for t in range(2))
                assert len(banks) == 64, (dt, h, half)


def test_swizzle_is_a_permutation_per_row():
    for r in range(32):
        assert sorted(c ^ row_swz(r) for c in range(16)) == list(range(16))
    assert np.unique([row_swz(r) for r in range(16)]).size == 16
