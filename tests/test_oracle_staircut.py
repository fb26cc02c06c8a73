"""Pins of the oracle's StairCut ("Drafters and tree verify", StairCut).

Worked examples by hand (tests/golden/staircut_examples.txt), then the rule's
structure: kept sets are closed under ancestors, cuts end only at the stair
points or the whole candidate, flat prices keep the largest cut, a price jump
between two stairs stops the cut below it, and the chain table prices a
chain.
"""
import os

import numpy as np
import pytest

from oracle import staircut as sc
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "staircut_examples.txt")


def _stairs(step9_16):
    p = np.zeros(33)
    p[1:9], p[9:17], p[17:25], p[25:33] = 10.0, step9_16, 14.0, 20.0
    return p


def test_worked_examples():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 2
    parents = [-1] + list(range(10))
    q = [0.0] + [0.8 ** d for d in range(1, 11)]
    for name, step, kept_nodes, score in rows:
        p = _stairs(float(step))
        kept, s = sc.staircut(parents, q, list(range(1, 11)), p, p, 1.0, 0.5)
        assert kept == list(range(int(kept_nodes) + 1)), name
        assert s == pytest.approx(float(score), rel=1e-9), name


def _random_candidate(n, seed):
    rng = np.random.default_rng(seed)
    parents = synth.random_tree(n, seed)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parents[i]] + 1
    q = [0.0] + [float(rng.uniform(0.3, 0.95) ** depth[i]) for i in range(1, n)]
    order = sorted(range(1, n), key=lambda i: -q[i] + 1e-9 * i)
    return [int(x) for x in parents], q, order


@pytest.mark.parametrize("seed", range(20))
def test_cut_structure(seed):
    n = 40 if seed % 2 else 20
    parents, q, order = _random_candidate(n, seed)
    rng = np.random.default_rng(100 + seed)
    price = np.cumsum(rng.uniform(0.0, 1.0, 33)) + 5.0
    kept, score = sc.staircut(parents, q, order, price, price * 0.9, 0.7, 0.3)
    s = set(kept)
    assert 0 in s
    for i in kept:                                # closed under ancestors
        assert i == 0 or parents[i] in s
    nodes = len(kept) - 1
    assert nodes <= 31
    # the kept set is an admission prefix's closure
    pref, found = {0}, nodes == 0
    for node in order:
        j = node
        while j >= 0:
            pref.add(j)
            j = parents[j]
        if pref == s:
            found = True
    assert found


def test_flat_prices_keep_the_largest_cut():
    parents, q, order = _random_candidate(30, 3)
    flat = np.full(33, 12.0)
    kept, _ = sc.staircut(parents, q, order, flat, flat, 1.0, 1.0)
    assert len(kept) == 30                        # whole candidate (29 nodes <= 31)
    parents, q, order = _random_candidate(45, 4)
    kept, _ = sc.staircut(parents, q, order, flat, flat, 1.0, 1.0)
    assert 24 <= len(kept) <= 32                  # the longest prefix within 31 nodes


def test_chain_table_prices_a_chain():
    parents = [-1] + list(range(10))
    q = [0.0] + [0.9] * 10
    tree = np.full(33, 100.0)
    chain = np.full(33, 10.0)
    chain[12:] = 1000.0
    kept, s = sc.staircut(parents, q, list(range(1, 11)), tree, chain, 0.0, 0.0)
    assert kept == list(range(11)) and s == pytest.approx((1 + 9.0) / 10.0)
