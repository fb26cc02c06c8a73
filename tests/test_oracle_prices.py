"""Verify prices for StairCut ("Drafters and tree verify", StairCut on
Flash-Next, and the shared price files): the oracle's plain price model
pinned to values worked by hand from the page's rules, and the library's
model (tv_prices_*, host code) against the oracle on random price files and
random measured rounds."""
import numpy as np
import pytest

from oracle import staircut as osc

POINTS = [(1024, "tree", 1, 10.0), (1024, "tree", 8, 12.0), (1024, "tree", 16, 14.0),
          (1024, "chain", 1, 9.0), (1024, "chain", 16, 12.0),
          (8192, "tree", 1, 20.0), (8192, "tree", 16, 30.0),
          (8192, "chain", 1, 19.0), (8192, "chain", 4, 18.0), (8192, "chain", 16, 25.0)]


def test_oracle_prices_by_hand():
    pm = osc.Prices(POINTS, step_ms=0.5)
    assert pm.context_class(500) == 1024 and pm.context_class(5000) == 1024
    assert pm.context_class(8192) == 8192 and pm.context_class(30000) == 8192
    t = pm.table(2000, "tree")
    assert t[1] == 10.0 and t[8] == 12.0 and t[16] == 14.0
    assert t[4] == pytest.approx(10.0 + 3 * 2.0 / 7)            # between 1 and 8: (12-10)/7 a row
    assert t[12] == pytest.approx(13.0)                          # halfway from 8 to 16
    assert t[20] == pytest.approx(14.0 + 4 * 0.5)                # past 16: step_ms a row
    assert t[0] == t[1]
    # no step_ms: the last two counts' slope, (14 - 12) / 8 a row
    assert osc.Prices(POINTS).table(2000, "tree")[20] == pytest.approx(15.0)
    # the dip to 18 ms at 4 rows is lifted: never falls with more rows
    c = pm.table(9000, "chain")
    assert c[2] == 19.0 and c[4] == 19.0 and c[16] == 25.0
    assert all(c[r] <= c[r + 1] for r in range(32))
    # a single listed count and no step: flat past it
    one = osc.Prices([(0, "tree", 4, 7.0)])
    assert one.table(100, "tree")[1] == 7.0 and one.table(100, "tree")[32] == 7.0
    # no file: 1 ms everywhere; a kind missing from the file: 1 ms too
    assert osc.Prices([]).table(4096, "tree") == [1.0] * 33
    assert osc.Prices([(0, "tree", 4, 7.0)]).table(100, "chain") == [1.0] * 33


def test_oracle_live_prices_by_hand():
    pm = osc.Prices(POINTS, step_ms=0.5)
    pm.observe(1024, "tree", 8, 20.0)                            # 12 + 0.1 (20 - 12)
    t = pm.table(1024, "tree")
    assert t[8] == pytest.approx(12.8)
    assert t[12] == pytest.approx(13.0 + 0.8)                    # shifted by the one offset, +0.8
    assert t[1] == pytest.approx(10.8) and t[16] == pytest.approx(14.8)
    pm.observe(1024, "tree", 8, 20.0)                            # 12.8 + 0.1 (20 - 12.8)
    assert pm.table(1024, "tree")[8] == pytest.approx(13.52)
    # 16 rows starts at its shifted price 14 + 1.52: 15.52 + 0.1 (10 - 15.52) = 14.968
    pm.observe(1024, "tree", 16, 10.0)
    t = pm.table(1024, "tree")
    # offsets 1.52 (8 rows) and 0.968 (16 rows): the others move by their mean, 1.244
    assert t[12] == pytest.approx(13.0 + 1.244)
    assert t[15] == pytest.approx(13.75 + 1.244)
    # 16 rows' live 14.968 lies below 15 rows' 14.994: lifted to it
    assert t[16] == pytest.approx(14.994)
    assert t[17] == pytest.approx(14.5 + 1.244)                  # past 16: step_ms a row, shifted
    assert pm.table(1024, "chain")[16] == 12.0                   # the other kind is untouched
    assert pm.table(8192, "tree")[16] == 30.0                    # and the other class


def _random_points(rng):
    pts = []
    for cls in rng.choice([0, 1024, 4096, 8192, 32768], size=rng.integers(0, 4), replace=False):
        for kind in ("chain", "tree"):
            if rng.random() < 0.2:
                continue
            rows = sorted(rng.choice(np.arange(1, 40), size=rng.integers(1, 6), replace=False))
            ms = np.cumsum(rng.uniform(-1.0, 4.0, len(rows))) + 10.0
            pts += [(int(cls), kind, int(r), float(m)) for r, m in zip(rows, ms)]
    return pts


@pytest.mark.parametrize("seed", range(40))
def test_native_prices_equal_oracle(seed):
    from greedy_draft_tree_amd.staircut import KINDS, PriceModel
    rng = np.random.default_rng(seed)
    pts = _random_points(rng)
    step = None if seed % 3 == 0 else float(rng.uniform(0.0, 1.0))
    ema = [0.1, 0.25, 1.0][seed % 3]
    table = {}
    for c, k, r, m in pts:
        table.setdefault(str(c), {}).setdefault(k, {})[str(r)] = m
    if step is not None:
        table["step_ms"] = step
    native = PriceModel(table, ema)
    orc = osc.Prices(pts, step_ms=step, ema=ema)
    ctxs = [0, 100, 1024, 3000, 8192, 20000, 40000]
    for i in range(25):
        for ctx in ctxs:
            assert native.class_of(ctx) == orc.context_class(ctx)
            for kind in KINDS:
                np.testing.assert_allclose(native.prices(ctx, kind), orc.table(ctx, kind), rtol=1e-12, atol=1e-12)
        ctx, kind, rows = int(rng.choice(ctxs)), KINDS[int(rng.integers(2))], int(rng.integers(1, 33))
        ms = float(rng.uniform(5.0, 40.0))
        native.observe(ctx, kind, rows, ms)
        orc.observe(ctx, kind, rows, ms)


def test_native_prices_reject_bad_input():
    from greedy_draft_tree_amd import TVError
    from greedy_draft_tree_amd.staircut import PriceModel
    with pytest.raises(TVError):
        PriceModel({"1024": {"tree": {"0": 1.0}}})                # a count below 1
    with pytest.raises(TVError):
        PriceModel({"1024": {"tree": {"4": float("nan")}}})
    with pytest.raises(TVError):
        PriceModel({}, ema=0.0)
    pm = PriceModel({})
    with pytest.raises(TVError):
        pm.observe(1024, "tree", 33, 5.0)
    with pytest.raises(TVError):
        pm.observe(1024, "tree", 4, float("inf"))
