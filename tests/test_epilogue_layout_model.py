"""CPU model of the grouped GEMM epilogues' lane exchanges (no GPU).

The MFMA accumulator fragment gives lane (g, c) = (lane // 16, lane % 16)
four consecutive output columns 4g..4g+3 of token row c.  The epilogues in
csrc/gemm.hip widen their global accesses in three ways:

  * pair_rows (v_permlane16_swap): for two fragments 16 columns apart, the
    16-lane rows 2k+1 of the first operand and 2k of the second trade places;
    lane group g then holds 8 consecutive columns 8*sig(g).. of the pair's 32,
    sig = (0, 2, 1, 3) (the gathered gate/up and the dH epilogues);
  * DPP row_ror:8 on top (dH): the two pairs of a 64-column quad trade
    8-lane halves, so lane (g, c) holds rows c%8 ("A") and 8 + c%8 ("B") at
    columns 32*(c >= 8) + 8*sig(g) -- each 16-byte access then covers 8 rows
    x 128 B;
  * the per-wave LDS slot (down, dX): 4-column pieces written at row c,
    column 16*ii + 4g of a 16 x 64 block, read back as chunk l%8 of rows l//8
    and 8 + l//8.

This test restates the hardware operations (the permlane16 swap semantics as
measured on gfx950: after the swap the first register holds rows (x0, y0,
x2, y2) and the second (x1, y1, x3, y3)) and checks that every output
element of the block is produced exactly once, at the right place, with the
right value.
"""
import numpy as np

LANES = 64


def frag(values, i):
    """Lane data of fragment i of a 16 x 64 block: lane (g, c) -> the 4 values
    at row c, columns 16 i + 4 g .. +3 (values[row, col])."""
    out = np.empty((LANES, 4), values.dtype)
    for lane in range(LANES):
        g, c = lane // 16, lane % 16
        out[lane] = values[c, 16 * i + 4 * g:16 * i + 4 * g + 4]
    return out


def permlane16_swap(x, y):
    """v_permlane16_swap_b32 on per-lane words (axis 0 = lane): odd 16-lane
    rows of x trade places with even rows of y."""
    xr, yr = x.reshape(4, 16, -1).copy(), y.reshape(4, 16, -1).copy()
    for k in (0, 2):
        xr[k + 1], yr[k] = y.reshape(4, 16, -1)[k].copy(), x.reshape(4, 16, -1)[k + 1].copy()
    return xr.reshape(x.shape), yr.reshape(y.shape)


def row_ror8(x):
    """DPP row_ror:8: lane c of each 16-lane row takes lane (c + 8) % 16."""
    xr = x.reshape(4, 16, -1)
    return np.roll(xr, -8, axis=1).reshape(x.shape)


SIG = [0, 2, 1, 3]


def test_permlane16_swap_model_matches_gfx950():
    """gfx950 gives a = [0..15, 100..115, 32..47, 132..147] and
    b = [16..31, 116..131, 48..63, 148..163] for a = lane, b = 100 + lane."""
    a = np.arange(64)[:, None]
    b = 100 + np.arange(64)[:, None]
    x, y = permlane16_swap(a, b)
    assert list(x[[0, 15, 16, 31, 32, 47, 48, 63], 0]) == [0, 15, 100, 115, 32, 47, 132, 147]
    assert list(y[[0, 15, 16, 31, 32, 47, 48, 63], 0]) == [16, 31, 116, 131, 48, 63, 148, 163]


def test_pair_rows_gives_each_lane_8_consecutive_columns():
    rng = np.random.default_rng(0)
    block = rng.standard_normal((16, 64))
    for m in range(2):   # the two pairs of the 64 columns
        x0, x1 = frag(block, 2 * m), frag(block, 2 * m + 1)
        lo, hi = permlane16_swap(x0, x1)
        seen = np.zeros((16, 32), int)
        for lane in range(LANES):
            g, c = lane // 16, lane % 16
            cols = 32 * m + 8 * SIG[g] + np.arange(8)
            got = np.concatenate([lo[lane], hi[lane]])
            np.testing.assert_array_equal(got, block[c, cols])
            seen[c, cols - 32 * m] += 1
        assert (seen == 1).all()


def test_dh_pair_then_ror8_covers_8_rows_x_64_columns_per_access():
    rng = np.random.default_rng(1)
    block = rng.standard_normal((16, 64))
    p = [permlane16_swap(frag(block, 0), frag(block, 1)),
         permlane16_swap(frag(block, 2), frag(block, 3))]
    s = [(row_ror8(a), row_ror8(b)) for a, b in p]
    lo = (np.arange(LANES) % 16) < 8
    # the kernel's selects: A = lo ? pair 0 : ror(pair 1), B = lo ? ror(pair 0) : pair 1
    A = np.where(lo[:, None], np.concatenate(p[0], 1), np.concatenate(s[1], 1))
    B = np.where(lo[:, None], np.concatenate(s[0], 1), np.concatenate(p[1], 1))
    seen = np.zeros((16, 64), int)
    rows_of_access = [set(), set()]
    for lane in range(LANES):
        g, c = lane // 16, lane % 16
        col = (0 if c < 8 else 32) + 8 * SIG[g] + np.arange(8)
        ra, rb = c % 8, 8 + c % 8
        np.testing.assert_array_equal(A[lane], block[ra, col])
        np.testing.assert_array_equal(B[lane], block[rb, col])
        seen[ra, col] += 1
        seen[rb, col] += 1
        rows_of_access[0].add(ra)
        rows_of_access[1].add(rb)
    assert (seen == 1).all()
    # each 16-byte access instruction covers 8 rows, each with all 64 columns
    assert rows_of_access == [set(range(8)), set(range(8, 16))]


def test_dh_row_partials_reduce_over_the_lanes_of_a_row():
    """d_row_scale partials: lane (g, c) sums its 8 columns of rows A and B;
    xor-shuffles over 8, 16 and 32 lanes then give every lane its row's
    total, and lanes 0..7 write rows c and 8 + c."""
    rng = np.random.default_rng(2)
    prod = rng.standard_normal((16, 64))   # h * gd per element
    pa = np.zeros(LANES)
    pb = np.zeros(LANES)
    for lane in range(LANES):
        g, c = lane // 16, lane % 16
        col = (0 if c < 8 else 32) + 8 * SIG[g] + np.arange(8)
        pa[lane] = prod[c % 8, col].sum()
        pb[lane] = prod[8 + c % 8, col].sum()
    for m in (8, 16, 32):
        pa = pa + pa[np.arange(LANES) ^ m]
        pb = pb + pb[np.arange(LANES) ^ m]
    for lane in range(8):
        np.testing.assert_allclose(pa[lane], prod[lane].sum())
        np.testing.assert_allclose(pb[lane], prod[8 + lane].sum())


def test_lds_slot_round_trip_covers_8_rows_x_128_bytes():
    """The down / dX slot: rows padded to 144 bytes; 8-byte writes of each
    fragment's 4-column piece, 16-byte reads of chunk l%8 of rows l//8 and
    8 + l//8."""
    pitch = 144
    rng = np.random.default_rng(3)
    block = rng.integers(0, 1 << 16, size=(16, 64), dtype=np.uint16)   # bf16 bits
    slot = np.full(16 * pitch // 2, -1, np.int64)                      # 2-byte cells
    writes = np.zeros(16 * pitch // 2, int)
    for ii in range(4):
        piece = frag(block, ii)
        for lane in range(LANES):
            g, c = lane // 16, lane % 16
            off = (c * pitch + (16 * ii + 4 * g) * 2) // 2
            assert (c * pitch + (16 * ii + 4 * g) * 2) % 8 == 0   # ds_write_b64 alignment
            slot[off:off + 4] = piece[lane]
            writes[off:off + 4] += 1
    assert writes.max() == 1 and writes.sum() == 16 * 64
    seen = np.zeros((16, 64), int)
    for lane in range(LANES):
        rr, ch = lane // 8, lane % 8
        for row in (rr, rr + 8):
            off = (row * pitch + ch * 16)
            assert off % 16 == 0                                           # ds_read_b128 alignment
            got = slot[off // 2:off // 2 + 8]
            np.testing.assert_array_equal(got, block[row, 8 * ch:8 * ch + 8])
            seen[row, 8 * ch:8 * ch + 8] += 1
    assert (seen == 1).all()
    assert 16 * pitch <= 2304   # the per-wave slot
