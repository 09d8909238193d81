"""LDS address maps of the two GEMM kernels (fwd.hip, dx.hip), enumerated on
the CPU.

The kernels place tiles, tables and codes in LDS with XOR swizzles, lane
permutations and byte-permute address arithmetic.  These tests restate each
map in Python and check, over every lane and index, what the kernels rely on:
writes and reads of one datum meet at the same address, every write map is a
bijection onto its buffer, and the accesses the LDS serves in one cycle (8
lanes for a 16-byte access, 32 lanes for 2- and 4-byte accesses; 32 banks of
4 bytes) hit distinct banks or the same dword.
"""

import random

import pytest

BANKS = 32


def bank(addr):
    return (addr // 4) % BANKS


def perm(s0, s1, sel):
    """v_perm_b32 for selector bytes 0..7: byte i of the result is byte
    sel_i of the 8-byte value {s0 (high), s1 (low)}."""
    src = s1 | (s0 << 32)
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        assert b < 8
        out |= ((src >> (8 * b)) & 0xFF) << (8 * i)
    return out


def conflict_free_16(addrs):
    """A 16-byte access of 8 lanes in one cycle: the 32 dwords are on 32 banks."""
    banks = [bank(a + 4 * d) for a in addrs for d in range(4)]
    return len(set(banks)) == len(banks)


def conflict_free_small(addrs):
    """2- or 4-byte accesses of 32 lanes: lanes on one bank read one dword."""
    seen = {}
    for a in addrs:
        b, dw = bank(a), a // 4
        if seen.setdefault(b, dw) != dw:
            return False
    return True


# ------------------------------------------------------------------ fwd.hip


def xswz(row, chunk):
    return row * 128 + ((chunk ^ (row & 7)) << 4)


def test_xswz_is_a_bijection_on_a_tile():
    offs = {xswz(r, c) for r in range(256) for c in range(8)}
    assert offs == set(range(0, 256 * 128, 16))


@pytest.mark.parametrize("ks", [0, 1])
@pytest.mark.parametrize("wm", [0, 1])
def test_fwd_a_fragment_reads_are_conflict_free(wm, ks):
    for i in range(8):
        addrs = []
        for lane in range(64):
            lr, kq = lane & 15, lane >> 4
            addrs.append(xswz(128 * wm + lr + 16 * i, 2 * kq + ks))
        for g in range(8):
            assert conflict_free_16(addrs[8 * g:8 * g + 8])


@pytest.mark.parametrize("wn", range(4))
def test_fwd_b_fragment_reads_are_conflict_free(wn):
    for ks in range(2):
        for j in range(4):
            addrs = [xswz(64 * wn + (l & 15) + 16 * j, 2 * (l >> 4) + ks) for l in range(64)]
            for g in range(8):
                assert conflict_free_16(addrs[8 * g:8 * g + 8])


@pytest.mark.parametrize("p", range(4))
def test_fwd_x_copy_lands_on_the_swizzled_tile(p):
    # instruction c of producer p fills 1 KB at (64p + 8c) * 128 + 16 * lane;
    # the lane fetches logical chunk (lane & 7) ^ (lane >> 3) of its row
    for c in range(8):
        for lane in range(64):
            row = 64 * p + 8 * c + (lane >> 3)
            logical = (lane & 7) ^ (lane >> 3)
            assert (64 * p + 8 * c) * 128 + 16 * lane == xswz(row, logical)


def fwd_table_base(row):
    return 32 * (row % 8) + 256 * (row // 8)


def test_fwd_tables_written_where_the_lookups_read_them():
    written = {}
    for p in range(4):
        for lane in range(64):
            off = 32 * (lane & 7) + 256 * (8 * p + (lane >> 3))
            written[64 * p + lane] = off
    assert sorted(written.values()) == list(range(0, 256 * 32, 32))
    for R in range(0, 256, 8):
        for dr in range(8):
            assert 256 * (R >> 3) + 32 * dr == written[R + dr] == fwd_table_base(R + dr)


def test_fwd_lookup_address_by_byte_permute():
    rnd = random.Random(7)
    stab = 0x1A00  # any 256-byte-aligned LDS address
    for _ in range(200):
        w = rnd.getrandbits(32)
        R = 8 * rnd.randrange(32)
        for dr in range(8):
            tab = stab + 256 * (R >> 3) + 32 * dr
            dr32x4 = dr * 0x20202020
            we = ((w << 1) & 0x1E1E1E1E) | dr32x4
            wo = ((w >> 3) & 0x1E1E1E1E) | dr32x4
            for j in range(4):
                code_e = (w >> (8 * j)) & 15
                code_o = (w >> (8 * j + 4)) & 15
                assert perm(tab, we, 0x07060500 | j) == tab + 2 * code_e
                assert perm(tab, wo, 0x07060500 | j) == tab + 2 * code_o


def test_fwd_lookups_are_conflict_free_for_any_codes():
    rnd = random.Random(3)
    for _ in range(200):
        R = 8 * rnd.randrange(32)
        codes = [rnd.randrange(16) for _ in range(64)]
        for half in range(2):
            addrs = []
            for lane in range(32 * half, 32 * half + 32):
                dr = lane >> 3
                addrs.append(fwd_table_base(R + dr) + 2 * codes[lane])
            assert conflict_free_small(addrs)


def test_fwd_w_tile_stores_are_conflict_free():
    for R in range(0, 256, 8):
        addrs = [xswz(R + (l >> 3), l & 7) for l in range(64)]
        assert sorted(addrs) == list(range(R * 128, (R + 8) * 128, 16))
        for g in range(8):
            assert conflict_free_16(addrs[8 * g:8 * g + 8])


# ------------------------------------------------------------------- dx.hip


def wswz(row, chunk):
    return row * 128 + ((chunk ^ ((row ^ (row >> 2)) & 7)) << 4)


def test_wswz_is_a_bijection_on_a_tile():
    offs = {wswz(r, c) for r in range(256) for c in range(8)}
    assert offs == set(range(0, 256 * 128, 16))


@pytest.mark.parametrize("wk", range(4))
def test_dx_b_fragment_reads_are_conflict_free(wk):
    for ks in range(2):
        for j in range(4):
            addrs = [wswz(64 * wk + (l & 15) + 16 * j, 2 * (l >> 4) + ks) for l in range(64)]
            for g in range(8):
                assert conflict_free_16(addrs[8 * g:8 * g + 8])


@pytest.mark.parametrize("sigma", range(8))
def test_dx_slice_store_identity_and_conflicts(sigma):
    for c in range(4):
        addrs = []
        for lane in range(64):
            rg, cg = lane >> 3, lane & 7
            st0 = (32 * sigma + 4 * cg) * 128 + ((rg ^ cg ^ (4 * (cg & 1))) << 4)
            a = (st0 ^ (16 * c)) + 128 * c
            assert a == wswz(32 * sigma + 4 * cg + c, rg)
            addrs.append(a)
        for g in range(8):
            assert conflict_free_16(addrs[8 * g:8 * g + 8])


def test_dx_code_transpose_meets_its_readers():
    # writer: lane l holds weight row l; its 2 bytes of column group pc go to
    # code_wbase ^ (pc << 4); reader (rg, cg) reads the 16-byte slot
    # 8rg + (cg ^ rg), whose byte 2i holds row 8rg + i
    where = {}
    for lane in range(64):
        wbase = (lane >> 3) * 128 + ((lane >> 3) << 4) + 2 * (lane & 7)
        for pc in range(8):
            off = wbase ^ (pc << 4)
            assert off not in where
            where[off] = (lane, pc)
    assert sorted(where) == list(range(0, 64 * 16, 2))
    for lane in range(64):
        rg, cg = lane >> 3, lane & 7
        slot = 8 * rg + (cg ^ rg)
        for i in range(8):
            assert where[16 * slot + 2 * i] == (8 * rg + i, cg)
    # the 16-bit writes of one instruction (fixed pc): 32 lanes per cycle
    for pc in range(8):
        for half in range(2):
            addrs = []
            for lane in range(32 * half, 32 * half + 32):
                wbase = (lane >> 3) * 128 + ((lane >> 3) << 4) + 2 * (lane & 7)
                addrs.append(wbase ^ (pc << 4))
            assert conflict_free_small(addrs)


def test_dx_table_writers_cover_the_tables_without_conflicts():
    halves = {}
    first, second = [], []
    for t in range(64):
        tb_rg = (t & 3) | ((t >> 1) & 4)
        tb_i = ((t >> 4) & 3) | (t & 4)
        tb_first = (t >> 2) & 1
        d = 256 * tb_i + 32 * tb_rg + 16 * tb_first
        row = 8 * tb_rg + tb_i
        # the table of row 8rg + i sits at 256i + 32rg; half tb_first first
        assert d & ~16 == 256 * tb_i + 32 * tb_rg
        halves[d] = (row, tb_first)
        halves[d ^ 16] = (row, 1 - tb_first)
        first.append(d)
        second.append(d ^ 16)
    assert sorted(halves) == list(range(0, 64 * 32, 16))
    assert len({r for r, _ in halves.values()}) == 64
    for g in range(8):
        assert conflict_free_16(first[8 * g:8 * g + 8])
        assert conflict_free_16(second[8 * g:8 * g + 8])


def test_dx_lookup_address_by_byte_permute():
    rnd = random.Random(11)
    stab = 0x4800
    for _ in range(200):
        cw = [rnd.getrandbits(32) for _ in range(4)]
        for rg in range(8):
            lb = stab + 32 * rg
            rg32x4 = rg * 0x20202020
            for p in range(4):
                we = ((cw[p] << 1) & 0x1E1E1E1E) | rg32x4
                wo = ((cw[p] >> 3) & 0x1E1E1E1E) | rg32x4
                for cp2 in range(2):
                    for h in range(2):
                        sel = 0x07060500 | (2 * h + cp2)
                        row = 2 * p + h  # row 8rg + row of the lane's group
                        for cc, src in ((0, we), (1, wo)):
                            col = 2 * cp2 + cc
                            code = (cw[p] >> (16 * h + 4 * col)) & 15
                            addr = perm(lb, src, sel) + 256 * row
                            assert addr == stab + 256 * row + 32 * rg + 2 * code


def test_dx_lookups_are_conflict_free_for_any_codes():
    # one lookup instruction: fixed (p, h, column); lane (rg, cg) reads the
    # table of row 8rg + 2p + h at 256(2p + h) + 32rg
    rnd = random.Random(5)
    for _ in range(200):
        codes = [rnd.randrange(16) for _ in range(64)]
        for p in range(4):
            for h in range(2):
                for half in range(2):
                    addrs = [256 * (2 * p + h) + 32 * (l >> 3) + 2 * codes[l]
                             for l in range(32 * half, 32 * half + 32)]
                    assert conflict_free_small(addrs)
