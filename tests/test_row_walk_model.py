"""CPU model of the persistent row kernels' unit walk (no GPU).

In k_scatter_rows_persist / k_gather_sum_persist (csrc/permute.hip) wave w of
a grid of W waves walks the (token, piece) units w, w + W, w + 2W, ... with a
(t, p) cursor advanced by W without a division (RowWalk), two units per loop
trip: the loads of unit n + 1 are issued before unit n's stores, and a trip
stores the unit it started with and the next one.  The loop is a do-while
that ends once the cursor passes the last token; units past the end have all
their accesses dropped.  This restates that control flow and checks that
every unit of every (ntok, pieces, W) is stored exactly once and that the
cursor equals divmod of the linear unit index at every step.
"""
import itertools


def walk_next(c, pieces, nw):
    t, p = c
    dq, dr = divmod(nw, pieces)
    p += dr
    t += dq
    if p >= pieces:
        p -= pieces
        t += 1
    return t, p


def stored_units(ntok, pieces, nw):
    """Units stored by the scatter's loop (the gather's has the same shape)."""
    out = []
    for w in range(nw):
        ca = divmod(w, pieces)
        lin = w
        while True:   # do { ... } while (ca.t < ntok)
            cb = walk_next(ca, pieces, nw)
            assert cb == divmod(lin + nw, pieces)
            if ca[0] < ntok:          # store(ca): dropped past the end
                out.append(ca)
            ca = walk_next(cb, pieces, nw)
            assert ca == divmod(lin + 2 * nw, pieces)
            if cb[0] < ntok:          # store(cb)
                out.append(cb)
            lin += 2 * nw
            if not ca[0] < ntok:
                break
    return out


def test_every_unit_is_stored_once():
    for ntok, pieces, nw in itertools.product((1, 2, 3, 7, 64, 257, 1000), (1, 2, 3, 6),
                                              (4, 8, 12, 36, 4096)):
        units = stored_units(ntok, pieces, nw)
        assert sorted(units) == [(t, p) for t in range(ntok) for p in range(pieces)], \
            (ntok, pieces, nw)


def test_gpt_oss_shape_trip_counts():
    """T = 4096 tokens of 2880 bf16 (two pieces of 192 chunks) on a grid of
    256 CUs x 4 blocks x 4 waves: two units per wave, one loop trip."""
    ntok, pieces, nw = 4096, 2, 256 * 4 * 4
    units = stored_units(ntok, pieces, nw)
    assert len(units) == len(set(units)) == ntok * pieces
    assert ntok * pieces / nw == 2
