"""CPU check of the wide-spread decode inputs used by the GPU parity tests:
each case puts the scores where its test says (no GPU)."""
import pytest

import spread_inputs as SI

CASES = [
    # mode, c_log2, bound on the largest excess of the last split over its first-tile floor
    ("late", 150, lambda e: e > 140),        # beyond fp32's exponent range: needs the exact maximum
    ("late", 90, lambda e: 70 < e < 120),    # above the first-pass limit of 64, below overflow
    ("late", 54, lambda e: 55 < e < 62.5),   # just under the limit: stays on the first pass
]


@pytest.mark.parametrize("mode,c,ok", CASES, ids=[f"{m}{c}" for m, c, _ in CASES])
@pytest.mark.parametrize("splits", [1, 3])
def test_late_maximum_cases(mode, c, ok, splits):
    w = SI.build(f"spread_{mode}{c}", mode, c)
    for b in range(w.B):
        ex = SI.excess_log2(w, b, splits)
        assert ok(ex[-1]), (b, ex)
        # the earlier splits hold only pushed-down rows: ordinary spreads
        assert all(e < 20 for e in ex[:-1]), (b, ex)


@pytest.mark.parametrize("splits", [1, 3])
def test_first_tile_maximum_case(splits):
    import numpy as np
    w = SI.build("spread_first200", "first", 200)
    for b in range(w.B):
        row = w.topk_indices[b]
        sel = np.unique(row[row >= 0])
        x = SI.scores_log2(w, b, sel)
        # for every head, every row after the first 32 lies at least 180 units
        # below the first rows' maximum: its probability underflows (2^-149 is
        # fp32's smallest subnormal)
        assert (x[:, 32:].max(axis=1) < x[:, :32].max(axis=1) - 180).all()
        # no split's first pass exceeds the limit
        assert max(SI.excess_log2(w, b, splits)) < 20


def test_pushed_rows_are_low_for_every_head():
    import numpy as np
    w = SI.build("spread_late150", "late", 150)
    for b in range(w.B):
        row = w.topk_indices[b]
        sel = np.unique(row[row >= 0])
        x = SI.scores_log2(w, b, sel)
        # pushed rows: about -150 for every head (rotary noise of a few units
        # on top); the three late rows stay ordinary
        assert (x[:, :-3] < -130).all() and (x[:, :-3] > -170).all()
        assert (np.abs(x[:, -3:]) < 20).all()


def test_split_ranges_cover_the_list():
    for count in (1, 7, 8, 33, 1000, 2048):
        for S in (1, 2, 3, 7):
            r = SI.split_ranges(count, S)
            assert r[0][0] == 0 and r[-1][1] == count
            assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
