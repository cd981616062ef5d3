"""Lane-level model of the MFMA kernels' index arithmetic (no GPU).

The GQA kernel (decode_spec.hip) and the MLA kernel (decode_mla.hip) move
tiles HBM -> LDS with direct-to-LDS loads that place 16-byte chunks at
XOR-swizzled positions, and read them back as MFMA operands (row-wise for
the scores, with a transposing 8-byte read for V^T: 16-bit elements, or int8
bytes widened in registers).  Each formula below is
the kernel's own, restated per lane; the tests check what has to hold between
them: the loads place every chunk of a tile exactly once, every read finds
the logical chunk it means, the two address paths of a tile load agree, and
the swizzles have the bank properties the kernels rely on.  A change to one
side of any pair (writer / reader) that the other side does not follow fails
here before any GPU run.
"""

import itertools

import pytest

TILE = 32  # tokens per tile (both kernels)


def swz(t):  # 3-bit swizzle of MLA rows (72 chunks)
    return (2 * (t & 3) + ((t >> 2) & 1)) ^ (2 * ((t >> 3) & 1))


def swz_i8(t):  # int8 GQA rows (8 chunks): the MLA swizzle, bit 1 also flipped by bit 4 of the row
    return swz(t) ^ (2 * ((t >> 4) & 1))


def swz16(t):  # 4-bit swizzle of 256-byte rows (16 chunks)
    return 8 * (t & 1) + 4 * ((t >> 1) & 1) + 2 * ((t >> 2) & 1) + (((t >> 3) ^ t) & 1)


# ----------------------------------------------------------------------------- GQA tile placement

def gqa_shape(i8):
    rb = 128 if i8 else 256  # bytes of one token row of one KV head
    cpr = rb // 16  # chunks per row
    lt = TILE * rb // 1024  # load instructions per K (or V) tile
    return rb, cpr, lt, (swz_i8 if i8 else swz16)


def gqa_placement(i8):
    """LDS chunk position P = 64 i + lane of a K (or V) tile -> (row, logical chunk)."""
    rb, cpr, lt, sw = gqa_shape(i8)
    out = {}
    for i in range(lt):
        for lane in range(64):
            P = 64 * i + lane
            t = P // cpr
            out[P] = (t, (P % cpr) ^ sw(t))
    return out


@pytest.mark.parametrize("i8", [False, True])
def test_gqa_tile_loads_place_every_chunk_once(i8):
    rb, cpr, lt, sw = gqa_shape(i8)
    place = gqa_placement(i8)
    assert sorted(place.values()) == [(t, c) for t in range(TILE) for c in range(cpr)]
    # the physical chunk of (t, c) inside its row is c ^ sw(t): the inverse used by every reader
    for P, (t, c) in place.items():
        assert P == t * cpr + (c ^ sw(t))


@pytest.mark.parametrize("nc", [16, 32])
def test_gqa_score_operand_reads(nc):
    """S^T A operand: lane (col, kg) at k-step ks reads channels KSTEP ks + 8 kg
    .. + 7 of token NC m + col (16-bit rows: one 16-byte chunk; int8 rows: one
    8-byte half of a chunk), at the position the tile loads put them."""
    kstep = 16 if nc == 32 else 32
    nks, nsa = 128 // kstep, TILE // nc
    for i8 in (False, True):
        rb, cpr, lt, sw = gqa_shape(i8)
        place = gqa_placement(i8)
        for lane, m, ks in itertools.product(range(64), range(nsa), range(nks)):
            kg, col = lane // nc, lane % nc
            t = nc * m + col
            c8 = (kstep * ks + 8 * kg) // 8  # 8-channel group of the row
            if i8:
                off = t * rb + 16 * ((c8 >> 1) ^ swz_i8(t)) + 8 * (c8 & 1)
                row, chunk = place[off // 16]
                assert (row, chunk, (off % 16) // 8) == (t, c8 >> 1, c8 & 1)  # 16 channels per int8 chunk
            else:
                off = t * rb + 16 * (c8 ^ swz16(t))
                assert off % 16 == 0 and place[off // 16] == (t, c8)


def pv_tokens(nc, kk, gq):
    """Tokens of k-slots 0..7 of the P^T operand in lane group gq (k-step kk):
    the S^T accumulator's token order, which the V^T operand must follow."""
    if nc == 32:  # 4 h + 0..3 and 8 + 4 h + 0..3 of the 16-token k-step, h = gq / 2
        first = 16 * kk + 4 * (gq >> 1)
        return [first + r for r in range(4)] + [first + 8 + r for r in range(4)]
    return [4 * gq + r for r in range(4)] + [16 + 4 * gq + r for r in range(4)]


def tr8_receive(addrs, byte_at):
    """ds_read_b64_tr_b8 on one 16-lane group: source lane s names 8 bytes at
    addrs[s] (row s / 2, columns 8 (s % 2) .. + 7 of the block); lane i
    receives column i, byte j from row j (measured with an in-bounds probe)."""
    return [[byte_at(addrs[2 * j + i // 8] + i % 8) for j in range(8)] for i in range(16)]


@pytest.mark.parametrize("nc", [16, 32])
def test_gqa_int8_transposing_v_reads(nc):
    """int8 V^T operand of PV MFMA n: lane i of group gq receives channel
    base + i (the MFMA row) for the 8 tokens of its k-slots, in slot order,
    from the int8 tile as the loads placed it."""
    place = gqa_placement(True)
    not_ = 128 // nc

    def byte_at(off):  # (token, channel) of LDS byte `off` of the int8 V tile
        t, c = place[off // 16]
        return (t, 16 * c + off % 16)

    for n in range(8):
        kk = n // not_ if nc == 32 else 0
        mt = n % not_ if nc == 32 else n
        for gq in range(4):
            addrs = []
            for s in range(16):
                j, e = s >> 1, s & 1
                t = (16 * kk + 8 * (j >> 2) + 4 * (gq >> 1) + (j & 3)) if nc == 32 else (16 * (j >> 2) + 4 * gq + (j & 3))
                c = 2 * mt + (gq & 1) if nc == 32 else mt
                addrs.append(t * 128 + 16 * (c ^ swz_i8(t)) + 8 * e)
            base = 32 * mt + 16 * (gq & 1) if nc == 32 else 16 * mt
            got = tr8_receive(addrs, byte_at)
            for i in range(16):
                assert got[i] == [(tok, base + i) for tok in pv_tokens(nc, kk, gq)], (nc, n, gq, i)


@pytest.mark.parametrize("nc", [16, 32])
def test_gqa_int8_transposing_v_reads_bank_groups(nc):
    """A 32-lane phase of that read (groups 2p, 2p + 1) names 16 rows x 16
    bytes that fall in 16 different 16-byte bank groups of a 256-byte bank
    sweep (128-byte rows alternate bank halves)."""
    not_ = 128 // nc
    for n in range(8):
        kk = n // not_ if nc == 32 else 0
        mt = n % not_ if nc == 32 else n
        for p in range(2):
            groups = set()
            for gq in (2 * p, 2 * p + 1):
                for j in range(8):
                    t = (16 * kk + 8 * (j >> 2) + 4 * (gq >> 1) + (j & 3)) if nc == 32 else (16 * (j >> 2) + 4 * gq + (j & 3))
                    c = 2 * mt + (gq & 1) if nc == 32 else mt
                    groups.add((t * 128 // 16 + (c ^ swz_i8(t))) % 16)
            assert len(groups) == 16, (nc, n, p)


def test_gqa_int8_old_swizzle_conflicts_in_the_transposing_read():
    """Without the row-bit-4 term, rows t and t + 16 of one 16-column group
    share a bank group (why the int8 swizzle has it)."""
    for gq in range(4):
        groups = [(t * 128 // 16 + (0 ^ swz(t))) % 16 for t in [4 * gq + r for r in range(4)] + [16 + 4 * gq + r for r in range(4)]]
        assert len(set(groups)) == 4


@pytest.mark.parametrize("nc", [16, 32])
def test_gqa_transposing_v_reads(nc):
    """V^T operand through ds_read_b64_tr_b16: in 16-lane group gq, source lane
    s = 4 r + q reads 4 channels (8 bytes) of one row; the group reads a
    4-row x 16-channel block, whose tokens are the k-slots the P^T operand
    assigns to the receiving lanes, and whose 16 channels are the MFMA rows
    (channel tile) of the output tile."""
    not_ = 128 // nc
    for tile in range(8):  # MFMA n of the PV loop
        kk = tile // not_ if nc == 32 else 0
        mt = tile % not_ if nc == 32 else tile
        tp = (mt & 1) if nc == 32 else (mt & 3)
        hi = (mt >> 1) if nc == 32 else (mt >> 2)
        for rd in range(2):
            for gq in range(4):
                rows, chans = set(), set()
                for s in range(16):
                    r, q = s >> 2, s & 3
                    t = (8 * rd + 4 * (gq >> 1) + r) if nc == 32 else (16 * rd + 4 * gq + r)
                    x = 8 * hi + (4 * (tp & 1) + 2 * (gq & 1) + (q >> 1) if nc == 32 else 2 * tp + (q >> 1))
                    off = t * 256 + 16 * (x ^ swz16(t)) + 8 * (q & 1) + 256 * 16 * kk
                    row = off // 256
                    pos = (off % 256) // 16
                    chunk = pos ^ swz16(row)  # the logical chunk stored there
                    rows.add(row)
                    chans.update(range(8 * chunk + 4 * (q & 1), 8 * chunk + 4 * (q & 1) + 4))
                base = 32 * mt + 16 * (gq & 1) if nc == 32 else 16 * mt
                assert chans == set(range(base, base + 16)), (nc, tile, rd, gq)
                if nc == 32:  # k-slots 4 h + 0..3 (rd 0) / 8 + 4 h + 0..3 (rd 1) of k-step kk, h = gq / 2
                    first = 16 * kk + 8 * rd + 4 * (gq >> 1)
                else:  # tokens 4 kg + 0..3 (rd 0) / 16 + 4 kg + 0..3 (rd 1), kg = gq
                    first = 16 * rd + 4 * gq
                assert rows == set(range(first, first + 4)), (nc, tile, rd, gq)


def gqa_rows(layout, i8, n_kv, g, b, tstart, end, table, bs, s_cap):
    """The per-lane path: byte address of every chunk load of the tile at tstart."""
    rb, cpr, lt, sw = gqa_shape(i8)
    out = []
    for i in range(lt):
        for lane in range(64):
            P = 64 * i + lane
            t = P // cpr
            c = (P % cpr) ^ sw(t)
            tok = min(tstart + t, end - 1)
            if layout in ("paged", "paged_bsh"):
                blk, slot = table[tok // bs], tok % bs
                row = (blk * bs + slot) * n_kv + g if layout == "paged_bsh" else (blk * n_kv + g) * bs + slot
            else:
                row = (b * s_cap + tok) * n_kv + g if layout == "bsnd" else (b * n_kv + g) * s_cap + tok
            out.append(row * rb + 16 * c)
    return out


def gqa_whole_tile(layout, i8, n_kv, g, b, tstart, table, bs, s_cap):
    """The whole-tile path: first row's address plus loff[i] (None when the tile is not whole)."""
    rb, cpr, lt, sw = gqa_shape(i8)
    token_major = layout in ("paged_bsh", "bsnd")
    stride = n_kv * rb if token_major else rb
    if layout in ("paged", "paged_bsh"):
        bi, u = tstart // bs, tstart % bs
        if u + TILE > bs:
            return None
        blk = table[bi]
        row0 = (blk * bs + u) * n_kv + g if token_major else (blk * n_kv + g) * bs + u
    else:
        row0 = (b * s_cap + tstart) * n_kv + g if token_major else (b * n_kv + g) * s_cap + tstart
    out = []
    for i in range(lt):
        for lane in range(64):
            P = 64 * i + lane
            t = P // cpr
            loff = t * stride + 16 * ((P % cpr) ^ sw(t))
            assert loff < 2 ** 32
            out.append(row0 * rb + loff)
    return out


@pytest.mark.parametrize("layout", ["paged", "paged_bsh", "bnsd", "bsnd"])
@pytest.mark.parametrize("i8", [False, True])
def test_gqa_whole_tile_path_matches_row_path(layout, i8):
    import random

    rng = random.Random(7)
    bs_choices = ([32, 64, 128, 256] if i8 else [16, 32, 64, 128, 256]) if layout.startswith("paged") else [0]
    checked = 0
    for _ in range(120):
        n_kv = rng.choice([1, 2, 8, 64])
        g, b = rng.randrange(n_kv), rng.randrange(3)
        bs = rng.choice(bs_choices)
        table = rng.sample(range(4000), 64)
        s_cap = 4096
        L = rng.randrange(33, 64 * bs if bs else s_cap)
        tstart = rng.randrange(0, L - TILE + 1)
        fast = gqa_whole_tile(layout, i8, n_kv, g, b, tstart, table, bs, s_cap)
        if fast is None:
            continue
        slow = gqa_rows(layout, i8, n_kv, g, b, tstart, L, table, bs, s_cap)
        assert fast == slow
        checked += 1
    assert checked > 40


# ----------------------------------------------------------------------------- MLA tile placement

MLA_CHUNKS = 72  # 1152-byte rows
MLA_ROWB = 1152


def test_mla_tile_loads_place_every_chunk_once():
    """Whole-tile offsets (computed once into LDS) and the per-row path
    address the same chunk for every load instruction and lane, and the 36
    instructions x 64 lanes cover the tile's 32 x 72 chunks once."""
    seen = []
    for ins in range(TILE * MLA_CHUNKS // 64):
        t0 = (64 * ins) // MLA_CHUNKS
        k1 = 64 * ins - MLA_CHUNKS * t0
        for lane in range(64):
            P = 64 * ins + lane
            t = P // MLA_CHUNKS
            whole = t * MLA_ROWB + 16 * ((P - MLA_CHUNKS * t) ^ swz(t))
            second = lane >= MLA_CHUNKS - k1
            pin = lane + k1 - (MLA_CHUNKS if second else 0)
            sw = swz(t0 + 1) if second else swz(t0)
            rowpath = (t0 + (1 if second else 0)) * MLA_ROWB + 16 * (pin ^ sw)
            assert whole == rowpath, (ins, lane)
            row, pos = whole // MLA_ROWB, (whole % MLA_ROWB) // 16
            assert pos // 8 == (pos ^ swz(row)) // 8  # the swizzle stays inside a group of 8 chunks
            seen.append((row, pos ^ swz(row)))
    assert sorted(seen) == [(t, c) for t in range(TILE) for c in range(MLA_CHUNKS)]


def test_mla_operand_reads():
    """S^T operand: lane (t = lane % 32, h = lane / 32) at k-step ks reads the
    logical chunk 2 ks + h of row t; V^T (transposing read): source lane
    s = 4 r + q of group g reads 4 channels of row 8 rd + 4 (g / 2) + r, and the
    group's 16 lanes cover 16 consecutive channels of 4 consecutive rows."""
    for lane in range(64):
        t, h = lane & 31, lane >> 5
        for ks in range(36):
            grp, j = ks // 4, ks % 4
            off = t * MLA_ROWB + 16 * ((2 * j + h) ^ swz(t)) + 128 * grp
            row, pos = off // MLA_ROWB, (off % MLA_ROWB) // 16
            assert row == t and pos ^ swz(t) == 2 * ks + h
    for kk, mt, rd, g in itertools.product(range(2), range(16), range(2), range(4)):
        rows, chans = set(), set()
        for s in range(16):
            r, q = s >> 2, s & 3
            odd = mt & 1
            t = 8 * rd + 4 * (g >> 1) + r
            x = 4 * odd + 2 * (g & 1) + (q >> 1)
            off = t * MLA_ROWB + 16 * (x ^ swz(t)) + 8 * (q & 1) + MLA_ROWB * 16 * kk + 128 * (mt >> 1)
            row, pos = off // MLA_ROWB, (off % MLA_ROWB) // 16
            chunk = pos ^ swz(row)
            rows.add(row)
            chans.update(range(8 * chunk + 4 * (q & 1), 8 * chunk + 4 * (q & 1) + 4))
        assert rows == set(range(16 * kk + 8 * rd + 4 * (g >> 1), 16 * kk + 8 * rd + 4 * (g >> 1) + 4))
        base = 32 * mt + 16 * (g & 1)
        assert chans == set(range(base, base + 16)), (kk, mt, rd, g)


# ----------------------------------------------------------------------------- swizzle properties

def test_swizzles_repeat_every_16_rows():
    """The 16-bit and MLA operand offsets add 16 rows per k-step as an
    immediate: valid only because those swizzles depend on the row modulo 16.
    The int8 swizzle repeats every 32 rows (a tile) and its reads take
    explicit offsets per k-step."""
    for t in range(64):
        assert swz(t) == swz(t + 16) and swz16(t) == swz16(t + 16)
        assert swz_i8(t) == swz_i8(t + 32) and swz_i8(t) == swz_i8(t + 16) ^ 2


def test_swz16_bank_properties():
    """256-byte rows start in the same bank; the 4-bit swizzle keeps each
    access of the GQA kernel free of two-way conflicts:
    16 consecutive rows -> 16 positions; 8 (from a multiple of 8) differ in
    swz16 / 2; 4 (from a multiple of 4) in swz16 / 4; rows 2j, 2j + 1 in parity."""
    for k in range(4):
        assert len({swz16(t) for t in range(16 * k, 16 * k + 16)}) == 16
    for k in range(8):
        assert len({swz16(t) >> 1 for t in range(8 * k, 8 * k + 8)}) == 8
    for k in range(16):
        assert len({swz16(t) >> 2 for t in range(4 * k, 4 * k + 4)}) == 4
    for j in range(32):
        assert swz16(2 * j) & 1 != swz16(2 * j + 1) & 1


def test_swz_spreads_rows_over_bank_groups():
    """3-bit swizzle: 8 consecutive rows (from a multiple of 8) take 8
    positions, and rows t and t + 8 differ; on 1152-byte MLA rows, which
    alternate bank halves, 16 consecutive rows' copies of one chunk then land
    in 16 different 16-byte bank groups (64 banks x 4 bytes).  The int8 GQA
    swizzle keeps both properties inside each 16-row window from a multiple of
    16 (the only rows its S^T operand reads take together), and on its
    128-byte rows those 16 rows' copies of one chunk also take 16 different
    bank groups."""
    for sw in (swz, swz_i8):
        for k in range(4):
            assert len({sw(t) for t in range(8 * k, 8 * k + 8)}) == 8
    for t in range(32):
        assert swz(t) != swz(t + 8)
    for t in [t for t in range(64) if t % 16 < 8]:
        assert swz_i8(t) != swz_i8(t + 8)
    for c in range(8):
        for k in range(2):
            assert len({(t * 128 // 16 + (c ^ swz_i8(t))) % 16 for t in range(16 * k, 16 * k + 16)}) == 16
    for c in range(MLA_CHUNKS):
        for k in range(2):
            groups = {((t * MLA_ROWB) // 16 + (c ^ swz(t))) % 16 for t in range(16 * k, 16 * k + 16)}
            assert len(groups) == 16, (c, k)
