"""The library's StairCut (tv_staircut, host code, no GPU) against the
oracle's plain reading, and the price model's lookup rules ("Drafters and
tree verify", StairCut; "StairCut on Flash-Next, and the shared price
files")."""
import numpy as np
import pytest

from oracle import staircut as osc
import synth


def _candidate(n, seed):
    rng = np.random.default_rng(seed)
    parents = [int(p) for p in synth.random_tree(n, seed)]
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parents[i]] + 1
    q = np.zeros(n, np.float32)
    for i in range(1, n):
        q[i] = np.float32(rng.uniform(0.2, 0.97) ** depth[i])
    order = [int(i) for i in rng.permutation(np.arange(1, n))] if seed % 3 == 0 else \
        sorted(range(1, n), key=lambda i: (-float(q[i]), i))
    return parents, q, order


def _prices(seed):
    rng = np.random.default_rng(1000 + seed)
    steps = np.repeat(rng.uniform(0.0, 4.0, 4), 8)
    p = np.zeros(33, np.float32)
    p[1:] = (8.0 + np.cumsum(steps) * (rng.random(32) < 0.3)).astype(np.float32)
    return np.maximum.accumulate(p).astype(np.float32)


@pytest.mark.parametrize("seed", range(60))
def test_cut_equals_oracle(seed):
    from greedy_draft_tree_amd.staircut import cut
    n = [1, 2, 5, 9, 17, 33, 40, 64, 120, 256][seed % 10]
    parents, q, order = _candidate(n, seed) if n > 1 else ([-1], np.zeros(1, np.float32), [])
    pt, pc = _prices(seed), (_prices(seed + 7) * np.float32(0.95)).astype(np.float32)
    draft, commit = float(np.float32(0.25 * (seed % 5))), float(np.float32(0.4))
    want, wscore = osc.staircut(parents, [float(x) for x in q], order, [float(x) for x in pt],
                                [float(x) for x in pc], draft, commit)
    got, gscore = cut(parents, q, order, pt, pc, draft, commit)
    assert got == want
    assert gscore == pytest.approx(wscore, rel=1e-6)


def test_cut_rejects_bad_input():
    from greedy_draft_tree_amd import TVError
    from greedy_draft_tree_amd.staircut import cut
    p = np.ones(33, np.float32)
    with pytest.raises(TVError):
        cut([-1, 0, 0], [0, 0.5, 0.5], [1, 1], p, p, 0, 0)          # not a permutation
    with pytest.raises(TVError):
        cut([-1, 2, 0], [0, 0.5, 0.5], [1, 2], p, p, 0, 0)          # parent after child
    with pytest.raises(TVError):
        cut([-1, 0], [0, -0.1], [1], p, p, 0, 0)                    # negative q
    bad = p.copy()
    bad[5] = np.inf
    with pytest.raises(TVError):
        cut([-1, 0], [0, 0.5], [1], bad, p, 0, 0)


# ------------------------------------------------------------ price model

FILE = {"1024": {"tree": {"1": 10.0, "8": 12.0, "16": 14.0}, "chain": {"1": 9.0, "16": 12.0}},
        "8192": {"tree": {"1": 20.0, "16": 30.0}, "chain": {"1": 19.0, "4": 18.0, "16": 25.0}},
        "step_ms": 0.5, "measured": "test"}


def test_price_classes_interpolation_and_extrapolation():
    from greedy_draft_tree_amd.staircut import PriceModel
    pm = PriceModel(FILE)
    assert pm.class_of(500) == 1024 and pm.class_of(5000) == 1024
    assert pm.class_of(8192) == 8192 and pm.class_of(30000) == 8192
    # between measured counts: linear
    assert pm.price(2000, "tree", 4) == pytest.approx(10.0 + 3 * 2.0 / 7)
    assert pm.price(2000, "tree", 12) == pytest.approx(13.0)
    # past the last count: step_ms a row
    assert pm.price(2000, "tree", 20) == pytest.approx(14.0 + 4 * 0.5)
    # without step_ms: the last two counts' slope
    f = dict(FILE)
    del f["step_ms"]
    assert PriceModel(f).price(2000, "tree", 20) == pytest.approx(14.0 + 4 * 0.25)
    # a price never falls with more rows (the file's dip at 4 rows is lifted)
    p = pm.prices(9000, "chain")
    assert np.all(np.diff(p[1:]) >= 0) and p[4] == pytest.approx(19.0)


def test_price_model_follows_live_prices_and_defaults():
    from greedy_draft_tree_amd.staircut import PriceModel
    pm = PriceModel(FILE)
    pm.observe(1024, "tree", 8, 20.0)
    assert pm.price(1024, "tree", 8) == pytest.approx(12.0 + 0.1 * 8.0)
    # unmeasured counts move by the learned offset (+0.8 here)
    assert pm.price(1024, "tree", 12) == pytest.approx(13.0 + 0.8)
    pm.observe(1024, "tree", 8, 20.0)
    assert pm.price(1024, "tree", 8) == pytest.approx(12.8 + 0.1 * 7.2)
    # the other class and kind are untouched
    assert pm.price(8192, "tree", 16) == pytest.approx(30.0)
    # no file: every count at 1 ms
    assert np.all(PriceModel().prices(4096, "tree")[1:] == 1.0)


def test_measure_shapes():
    from greedy_draft_tree_amd.staircut import _tree_shape
    for r in range(1, 33):
        for kind in ("chain", "tree"):
            p = _tree_shape(r, kind)
            assert len(p) == r and p[0] == -1 and all(0 <= p[i] < i for i in range(1, r))


def test_measured_prices_load_and_cut():
    """The committed MI355X price file loads; on its nearly flat prices the
    cut keeps a whole 31-node candidate of fair path probabilities."""
    import json
    import os
    import re
    from greedy_draft_tree_amd.staircut import PriceModel, cut
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                        "verify_prices_c1_c2.md")
    blocks = re.findall(r"```json\n(.*?)\n```", open(path).read(), flags=re.S)
    assert len(blocks) == 2
    for b in blocks:
        pm = PriceModel(json.loads(b))
        for ctx in (1024, 8192, 32768, 65536):
            for kind in ("chain", "tree"):
                p = pm.prices(ctx, kind)
                assert np.all(np.diff(p[1:]) >= 0) and p[1] > 0
        parents, q, order = _candidate(32, 5)
        keep, _ = cut(parents, np.maximum(q, np.float32(0.3)), order, pm.prices(1024, "tree"),
                      pm.prices(1024, "chain"), 0.5, 0.1)
        assert len(keep) == 32
