"""Index algebra the HIP kernels rely on, checked exhaustively on the host.

The device helpers cannot be called from Python, so each is restated here from
its definition in gated_delta_rule_41_amd/csrc (kda_internal.h: kt_off,
KtFrag; kda_device.h: perm32, col4) and checked for the properties the kernels
assume.  A change to one of those helpers has to keep these properties; the
GPU parity tests then check the kernels end to end.
"""
import itertools

KCHUNK = 64


def kt_off(c, pos):
    # transposed tile [row c][64 positions], 16-byte groups XOR-swizzled by (c ^ c>>3) & 7
    return c * KCHUNK + ((((pos >> 3) ^ (c ^ (c >> 3))) & 7) << 3) + (pos & 7)


def ktfrag_at(qg, cl, m, kk):
    # four lane values b[x] = 64 cl + ((g0 ^ 2x) << 3), g0 = (qg ^ cl ^ (cl >> 3)) & 7
    g0 = (qg ^ cl ^ (cl >> 3)) & 7
    b = [KCHUNK * cl + ((g0 ^ (2 * x)) << 3) for x in range(4)]
    return b[(((4 * kk) ^ (2 * m)) & 7) >> 1] + 16 * KCHUNK * m


def perm32(k):
    kk = k & 31
    return (k & ~31) | (((kk >> 2) & 3) << 3) | ((kk >> 4) << 2) | (kk & 3)


def v_perm_b32(s0, s1, sel):
    # byte k of the result: selector byte b picks byte b of S1 (b < 4) or byte b-4 of S0 (b < 8)
    src = list(s1.to_bytes(4, "little")) + list(s0.to_bytes(4, "little"))
    return bytes(src[(sel >> (8 * k)) & 0xFF] for k in range(4))


def test_kt_off_is_a_bijection_that_keeps_16_byte_groups():
    seen = set()
    for c in range(128):            # up to dk = 128 rows
        for pos in range(KCHUNK):
            o = kt_off(c, pos)
            assert c * KCHUNK <= o < (c + 1) * KCHUNK       # stays in its own row
            seen.add(o)
        for g in range(8):          # each aligned group of 8 positions maps to 8 contiguous elements
            base = kt_off(c, 8 * g)
            assert base % 8 == 0
            assert [kt_off(c, 8 * g + j) for j in range(8)] == list(range(base, base + 8))
    assert len(seen) == 128 * KCHUNK


def test_kt_off_spreads_a_fragment_read_over_all_groups():
    # the 16 rows an A-fragment read touches (row 16m + cl, fixed position group) hit
    # all eight 16-byte groups twice: no two lanes of a half-wave share a group slot
    for m in range(8):
        for pos in range(0, KCHUNK, 8):
            groups = [(kt_off(16 * m + cl, pos) % KCHUNK) // 8 for cl in range(16)]
            assert sorted(groups) == sorted(list(range(8)) * 2)


def test_ktfrag_equals_kt_off_for_every_lane_and_step():
    for qg, cl, m, kk in itertools.product(range(4), range(16), range(8), range(2)):
        assert ktfrag_at(qg, cl, m, kk) == kt_off(16 * m + cl, 32 * kk + 8 * qg), (qg, cl, m, kk)


def test_perm32_matches_stacked_accumulator_fragments():
    # a k32 fragment made of two stacked 16x16 accumulator blocks gives lane group qg the
    # logical k {4qg..4qg+3, 16+4qg..16+4qg+3}; perm32 must place them at 8qg..8qg+7
    for base in (0, 32, 64, 96):
        assert sorted(perm32(base + k) for k in range(32)) == list(range(base, base + 32))
        for qg in range(4):
            ks = [base + 4 * qg + j for j in range(4)] + [base + 16 + 4 * qg + j for j in range(4)]
            assert [perm32(k) for k in ks] == list(range(base + 8 * qg, base + 8 * qg + 8))


def test_col4_selectors_take_one_column_of_a_bf16_block():
    # rows r0..r3 of four 16-bit values each, as two little-endian dwords per row
    rows = [[(0x1000 * (r + 1) + j) & 0xFFFF for j in range(4)] for r in range(4)]
    words = [[row[0] | (row[1] << 16), row[2] | (row[3] << 16)] for row in rows]
    for j in range(4):
        sel = 0x07060302 if j & 1 else 0x05040100
        lo = v_perm_b32(words[1][j >> 1], words[0][j >> 1], sel)
        hi = v_perm_b32(words[3][j >> 1], words[2][j >> 1], sel)
        got = [int.from_bytes(lo[0:2], "little"), int.from_bytes(lo[2:4], "little"),
               int.from_bytes(hi[0:2], "little"), int.from_bytes(hi[2:4], "little")]
        assert got == [rows[r][j] for r in range(4)], j
