"""LDS address maps of the two GEMM kernels (fwd.hip, dx.hip), enumerated on
the CPU.

The kernels place tiles, tables and codes in LDS with XOR swizzles, lane
permutations and byte-permute address arithmetic.  These tests restate each
map in Python and check, over every lane and index, what the kernels rely on:
writes and reads of one datum meet at the same address, every write map is a
bijection onto its buffer, and the 2-byte table lookups of one half-wave hit
distinct banks or the same dword (the gfx950 LDS serves 2- and 4-byte
accesses 32 lanes per clock on 32 banks of 4 bytes).

The 16-byte accesses follow no such simple rule on gfx950: reads stream at
256 bytes per clock for some lane patterns and half that for others, and
writes at about 80 bytes per clock whatever the pattern.  The chunk
permutations of the tiles were chosen by timing the kernels' exact read
patterns on the hardware; the tests below pin the permutations themselves
(the fragment reads see, in every 16-row group, the measured arrangement).
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


def conflict_free_small(addrs):
    """2- or 4-byte accesses of 32 lanes: lanes on one bank read one dword."""
    seen = {}
    for a in addrs:
        b, dw = bank(a), a // 4
        if seen.setdefault(b, dw) != dw:
            return False
    return True


# ------------------------------------------------------------------ fwd.hip


def rsw(r):
    """Bits 0 and 1 of r swapped (r < 8)."""
    return ((r >> 1) & 1) | ((r & 1) << 1) | (r & 4)


def xswz(row, chunk):
    return row * 128 + ((chunk ^ rsw(row & 7)) << 4)


def fragment_slots(swz, base, ks):
    """(row parity, physical chunk) of each lane of an MFMA fragment read:
    lane l reads row base + (l & 15) at chunk 2(l >> 4) + ks."""
    out = []
    for l in range(64):
        a = swz(base + (l & 15), 2 * (l >> 4) + ks)
        out.append(((a // 128) & 1, (a % 128) // 16))
    return out


# The chunk permutation of every 16-row group that the fragment reads met at
# the full read rate when timed: row r (r = 0..15 of the group) puts logical
# chunk c at physical c ^ P[r].
MEASURED_FAST_X = [0, 2, 1, 3, 4, 6, 5, 7, 0, 2, 1, 3, 4, 6, 5, 7]
MEASURED_FAST_W = [0, 0, 2, 2, 4, 4, 6, 6, 1, 1, 3, 3, 5, 5, 7, 7]


def test_xswz_is_a_bijection_on_a_tile():
    offs = {xswz(r, c) for r in range(256) for c in range(8)}
    assert offs == set(range(0, 256 * 128, 16))


@pytest.mark.parametrize("ks", [0, 1])
@pytest.mark.parametrize("wm", [0, 1])
def test_fwd_a_fragment_reads_use_the_measured_permutation(wm, ks):
    for i in range(8):
        for lane in range(64):
            lr, kq = lane & 15, lane >> 4
            a = xswz(128 * wm + lr + 16 * i, 2 * kq + ks)
            assert a == (128 * wm + lr + 16 * i) * 128 + (((2 * kq + ks) ^ MEASURED_FAST_X[lr]) << 4)


@pytest.mark.parametrize("wn", range(4))
def test_fwd_b_fragment_reads_are_conflict_free(wn):
    for ks in range(2):
        for j in range(4):
            for l in range(64):
                row = 64 * wn + (l & 15) + 16 * j
                assert xswz(row, 2 * (l >> 4) + ks) == row * 128 + (((2 * (l >> 4) + ks) ^ MEASURED_FAST_X[l & 15]) << 4)


@pytest.mark.parametrize("p", range(4))
def test_fwd_x_copy_lands_on_the_swizzled_tile(p):
    # instruction c of producer p fills 1 KB at (64p + 8c) * 128 + 16 * lane;
    # the lane fetches logical chunk (lane & 7) ^ sw(lane >> 3) of its row
    for c in range(8):
        for lane in range(64):
            row = 64 * p + 8 * c + (lane >> 3)
            logical = (lane & 7) ^ rsw(lane >> 3)
            assert (64 * p + 8 * c) * 128 + 16 * lane == xswz(row, logical)


def fwd_row_table(vals):
    """The producer lane's byte planes: L[g] = low bytes of values 4g..4g+3,
    H[g] the high bytes, from the packed pairs d[j] = v[2j] | v[2j+1] << 16."""
    d = [vals[2 * j] | (vals[2 * j + 1] << 16) for j in range(8)]
    L = [perm(d[2 * g + 1], d[2 * g], 0x06040200) for g in range(4)]
    H = [perm(d[2 * g + 1], d[2 * g], 0x07050301) for g in range(4)]
    return L, H


def fwd_look(c, T):
    s7 = c & 0x07070707
    sel = ((c >> 1) & 0x04040404) | 0x03020100
    return perm(perm(T[3], T[2], s7), perm(T[1], T[0], s7), sel)


def fwd_decode8(w, L, H):
    ev, od = w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F
    le, he, lo, ho = fwd_look(ev, L), fwd_look(ev, H), fwd_look(od, L), fwd_look(od, H)
    e01, e23 = perm(he, le, 0x05010400), perm(he, le, 0x07030602)
    o01, o23 = perm(ho, lo, 0x05010400), perm(ho, lo, 0x07030602)
    return [perm(o01, e01, 0x05040100), perm(o01, e01, 0x07060302),
            perm(o23, e23, 0x05040100), perm(o23, e23, 0x07060302)]


def check_decode(vals, w):
    L, H = fwd_row_table(vals)
    out = fwd_decode8(w, L, H)
    codes = [(w >> (4 * k)) & 15 for k in range(8)]  # element 2b: low nibble of byte b
    for i in range(4):
        assert out[i] == vals[codes[2 * i]] | (vals[codes[2 * i + 1]] << 16), (hex(w), i)


def test_fwd_register_decode_gives_the_table_values():
    # every code in every one of the 8 positions of a dword (the other seven
    # random), distinct random 16-bit table values, and all-equal dwords
    rnd = random.Random(11)
    for _ in range(40):
        vals = [rnd.getrandbits(16) for _ in range(16)]
        for pos in range(8):
            for code in range(16):
                w = rnd.getrandbits(32) & ~(15 << (4 * pos)) | (code << (4 * pos))
                check_decode(vals, w)
        for code in range(16):
            check_decode(vals, code * 0x11111111)


def test_fwd_producer_stores_cover_the_w_tile():
    # lane l of producer p stores the 8 chunks of tile row 64p + l
    addrs = sorted(xswz(64 * p + lane, j) for p in range(4) for lane in range(64) for j in range(8))
    assert addrs == list(range(0, 256 * 128, 16))


@pytest.mark.parametrize("p", range(4))
def test_fwd_tall_x_copy_lands_on_the_swizzled_tile(p):
    # 512 x 128 tile: producer p copies X rows [128p, +128) with 16
    # instructions of 8 rows; every row's 8 chunks land once
    seen = set()
    for c in range(16):
        for lane in range(64):
            row = 128 * p + 8 * c + (lane >> 3)
            logical = (lane & 7) ^ rsw(lane >> 3)
            a = (128 * p + 8 * c) * 128 + 16 * lane
            assert a == xswz(row, logical)
            seen.add(a)
    assert sorted(seen) == list(range(128 * p * 128, 128 * (p + 1) * 128, 16))


def test_fwd_tall_producer_stores_cover_the_w_tile():
    # 512 x 128 tile: lane l of producer p owns row 32p + l % 32 and stores
    # its chunks 4h .. 4h + 3, h = l // 32 (16 of the row's 32 bytes of codes)
    addrs = sorted(xswz(32 * p + lane % 32, 4 * (lane // 32) + jj)
                   for p in range(4) for lane in range(64) for jj in range(4))
    assert addrs == list(range(0, 128 * 128, 16))


@pytest.mark.parametrize("wave", range(8))
def test_fwd_tall_fragment_reads_stay_in_the_tiles(wave):
    # 4 x 2 MFMA waves of 128 x 64: A rows below 512, B rows below 128, the
    # same measured chunk arrangement as the square tile
    wm, wn = wave // 2, wave % 2
    for ks in range(2):
        for l in range(64):
            for i in range(8):
                ra = 128 * wm + (l & 15) + 16 * i
                assert ra < 512
                assert xswz(ra, 2 * (l >> 4) + ks) == ra * 128 + (((2 * (l >> 4) + ks) ^ MEASURED_FAST_X[l & 15]) << 4)
            for j in range(4):
                rb = 64 * wn + (l & 15) + 16 * j
                assert rb < 128


# ------------------------------------------------------------------- dx.hip


def wsw(row):
    """r3 | r1 << 1 | r2 << 2 for bits r_i of row."""
    return ((row >> 3) & 1) | (row & 2) | (row & 4)


def wswz(row, chunk):
    return row * 128 + ((chunk ^ wsw(row)) << 4)


def dq_rg(l):
    """Row group of lane l in a dequantization slice (lane bits 1, 2, 5)."""
    return ((l >> 1) & 3) | ((l >> 3) & 4)


def dq_cg(l):
    """Column group of lane l in a dequantization slice (lane bits 0, 3, 4)."""
    return (l & 1) | ((l >> 2) & 6)


def test_dq_lane_map_is_a_bijection():
    assert {(dq_rg(l), dq_cg(l)) for l in range(64)} == {(rg, cg) for rg in range(8) for cg in range(8)}


@pytest.mark.parametrize("sigma", range(8))
def test_dx_slice_stores_of_8_lanes_hit_8_chunk_positions(sigma):
    # one store instruction (column c of the lanes' 4): each run of 8
    # consecutive lanes writes 8 distinct 16-byte chunk positions of the
    # 128-byte rows (the map that took the measured LDS bank conflicts of
    # the dX GEMM from 256 to 32 cycles per step)
    for c in range(4):
        for g in range(8):
            chunks = {(wswz(32 * sigma + 4 * dq_cg(l) + c, dq_rg(l)) % 128) // 16 for l in range(8 * g, 8 * g + 8)}
            assert len(chunks) == 8


def test_wswz_is_a_bijection_on_a_tile():
    offs = {wswz(r, c) for r in range(256) for c in range(8)}
    assert offs == set(range(0, 256 * 128, 16))


@pytest.mark.parametrize("wk", range(4))
def test_dx_b_fragment_reads_use_the_measured_permutation(wk):
    for ks in range(2):
        for j in range(4):
            for l in range(64):
                row = 64 * wk + (l & 15) + 16 * j
                assert wswz(row, 2 * (l >> 4) + ks) == row * 128 + (((2 * (l >> 4) + ks) ^ MEASURED_FAST_W[l & 15]) << 4)


def test_dx_a_tile_uses_the_forward_permutation():
    for row in range(256):
        for c in range(8):
            assert xswz(row, c) == row * 128 + ((c ^ MEASURED_FAST_X[row & 15]) << 4)


@pytest.mark.parametrize("p", range(4))
def test_dx_at2_copy_lands_on_the_swizzled_tile(p):
    # copy_at: instruction c fills 1 KB at (64p + 8c) * 128 + 16 * lane with
    # logical chunk (lane & 7) ^ wsw(row) of row 64p + 8c + (lane >> 3)
    seen = set()
    for c in range(8):
        for lane in range(64):
            row = 64 * p + 8 * c + (lane >> 3)
            lch = (lane & 7) ^ wsw(row)
            assert (64 * p + 8 * c) * 128 + 16 * lane == wswz(row, lch)
            seen.add((row, lch))
    assert len(seen) == 512


@pytest.mark.parametrize("sigma", range(8))
def test_dx_slice_store_identity(sigma):
    seen = set()
    for c in range(4):
        for lane in range(64):
            rg, cg = dq_rg(lane), dq_cg(lane)
            st0 = (32 * sigma + 4 * cg) * 128 + ((rg ^ ((cg >> 1) & 1) ^ (4 * (cg & 1))) << 4)
            a = (st0 ^ (16 * (c & 2))) + 128 * c
            assert a == wswz(32 * sigma + 4 * cg + c, rg)
            seen.add(a)
    assert sorted(seen) == list(range(32 * sigma * 128, (32 * sigma + 32) * 128, 16))


def test_dx_code_transpose_meets_its_readers():
    # writer: lane l (m = l & 31, h = l >> 5) holds 16 bytes of weight rows
    # 2m and 2m + 1 for slice h; per column group pc it stores one dword (2
    # bytes of row 2m, then 2 bytes of row 2m + 1) at byte 4(m & 3) of slot
    # 8rg + (pc ^ rg), rg = m >> 2.  Reader (rg, cg) reads the 16-byte slot
    # 8rg + (cg ^ rg), whose byte 2i holds row 8rg + i.
    for h in range(2):
        where = {}
        for lane in range(32 * h, 32 * h + 32):
            m = lane & 31
            rg = m >> 2
            for pc in range(8):
                off = rg * 128 + (((pc ^ rg) & 7) << 4) + 4 * (m & 3)
                for half, row in ((0, 2 * m), (1, 2 * m + 1)):
                    assert off + 2 * half not in where
                    where[off + 2 * half] = (row, pc)
        assert sorted(where) == list(range(0, 64 * 16, 2))
        for lane in range(64):
            rg, cg = dq_rg(lane), dq_cg(lane)
            slot = 8 * rg + (cg ^ rg)
            for i in range(8):
                assert where[16 * slot + 2 * i] == (8 * rg + i, cg)
    # the 4-byte writes of one instruction (fixed pc): 32 lanes per cycle
    for pc in range(8):
        for half in range(2):
            addrs = []
            for lane in range(32 * half, 32 * half + 32):
                m = lane & 31
                rg = m >> 2
                addrs.append(rg * 128 + (((pc ^ rg) & 7) << 4) + 4 * (m & 3))
            assert conflict_free_small(addrs)
    # the byte permute puts row 2m's 2 bytes low and row 2m + 1's high
    rnd = random.Random(3)
    for _ in range(100):
        c0, c1 = rnd.getrandbits(32), rnd.getrandbits(32)
        for odd, sel in ((0, 0x05040100), (1, 0x07060302)):
            w = perm(c1, c0, sel)
            assert w & 0xFFFF == (c0 >> (16 * odd)) & 0xFFFF
            assert w >> 16 == (c1 >> (16 * odd)) & 0xFFFF


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
                    addrs = [256 * (2 * p + h) + 32 * dq_rg(l) + 2 * codes[l]
                             for l in range(32 * half, 32 * half + 32)]
                    assert conflict_free_small(addrs)
