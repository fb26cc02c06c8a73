"""Pins of the oracle's lookup drafter ("Drafters and tree verify", The lookup
drafter).

* hand-worked examples (tests/golden/lookup_examples.txt);
* a closed form: on a periodic text the tree is one chain, the periodic
  continuation, with q(d) = (V - ceil(d / P) + 1) / V for V = floor((L - o) / P)
  votes of period P;
* every kept node's q against a direct count of the occurrences followed by
  its path (no tree building), and the order used against the absence of any
  occurrence one order longer;
* every text of length <= 7 over three tokens: the output is a tree in
  depth-first pre-order with distinct sibling tokens, closed under ancestors,
  admitted best first.
"""
import itertools
import math
import os

import numpy as np
import pytest

from oracle.lookup import lookup_draft

GOLD = os.path.join(os.path.dirname(__file__), "golden", "lookup_examples.txt")


def _golden():
    out = []
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        f = [x.strip() for x in line.split("|")]
        ints = lambda s: [] if s == "-" else [int(x) for x in s.split()]
        q = [float(np.float32(int(a) / int(b))) for a, b in (x.split("/") for x in f[5].split())]
        out.append((f[0], ints(f[1]), ints(f[2]), ints(f[3]), ints(f[4]), q, ints(f[6]), int(f[7]), int(f[8])))
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c[0])
def test_hand_worked_examples(case):
    _, text, prm, parents, tokens, q, order, o, votes = case
    got = lookup_draft(text, *prm)
    assert got == (parents, tokens, q, order, o, votes)


@pytest.mark.parametrize("P,L,o,depth,nodes", [(3, 20, 4, 31, 31), (5, 23, 8, 31, 31), (4, 40, 8, 7, 31),
                                               (7, 30, 2, 31, 5), (2, 11, 3, 31, 31)])
def test_periodic_text_closed_form(P, L, o, depth, nodes):
    text = [i % P for i in range(L)]
    parents, tokens, q, order, got_o, V = lookup_draft(text, 2, o, depth, nodes)
    assert got_o == o and V == (L - o) // P
    n = min(depth, V * P, nodes)
    assert parents == [-1] + list(range(n))
    assert tokens == [(L - 1 + d) % P for d in range(n + 1)]
    want = [1.0] + [float(np.float32((V - math.ceil(d / P) + 1) / V)) for d in range(1, n + 1)]
    assert q == want
    assert order == list(range(1, n + 1))
    # with a continuation rate a level: the same tree, q(d) times rho^d
    rho = 0.625
    p2, t2, q2, o2, _, _ = lookup_draft(text, 2, o, depth, nodes, rho)
    assert (p2, t2, o2) == (parents, tokens, order)
    assert q2 == [1.0] + [float(np.float32((V - math.ceil(d / P) + 1) / V * rho ** d)) for d in range(1, n + 1)]


def _path(parents, tokens, i):
    out = []
    while i > 0:
        out.append(tokens[i])
        i = parents[i]
    return out[::-1]


def _check_against_direct_count(text, mn, mx, depth, nodes):
    parents, tokens, q, order, o, V = lookup_draft(text, mn, mx, depth, nodes)
    L = len(text)
    suffix = lambda k: tuple(text[L - k:])
    grams = lambda k: {tuple(text[p:p + k]) for p in range(0, L - k)}   # occurrences ending before the text
    if o == 0:
        assert V == 0 and parents == [-1]
        for k in range(mn, min(mx, L - 1) + 1):
            assert suffix(k) not in grams(k)
        return
    assert mn <= o <= mx and suffix(o) in grams(o)
    for k in range(o + 1, min(mx, L - 1) + 1):
        assert suffix(k) not in grams(k)
    starts = [p for p in range(L - o) if tuple(text[p:p + o]) == suffix(o)]
    assert V == len(starts)
    for i in range(1, len(parents)):
        path = _path(parents, tokens, i)
        d = len(path)
        assert d <= depth
        c = sum(1 for p in starts if p + o + d <= L and text[p + o:p + o + d] == path)
        assert c > 0 and q[i] == float(np.float32(c / V)), (text, i, path)


def test_random_texts_against_direct_count():
    rng = np.random.default_rng(11)
    for t in range(300):
        L = int(rng.integers(2, 90))
        alpha = int(rng.integers(2, 6))
        text = [int(x) for x in rng.integers(0, alpha, L)]
        mn = int(rng.integers(1, 4))
        mx = int(rng.integers(mn, 10))
        _check_against_direct_count(text, mn, mx, int(rng.integers(1, 12)), int(rng.integers(0, 40)))


def _key_of(parents, tokens, q, i):
    return (-q[i], len(_path(parents, tokens, i)), _path(parents, tokens, i))


def test_every_tiny_text_gives_a_best_first_tree():
    for L in range(1, 8):
        for text in itertools.product(range(3), repeat=L):
            for nodes in (1, 3, 31):
                parents, tokens, q, order, o, V = lookup_draft(list(text), 2, 8, 4, nodes)
                n = len(parents)
                assert tokens[0] == text[-1] and q[0] == 1.0
                assert n - 1 <= nodes and sorted(order) == list(range(1, n))
                for i in range(1, n):
                    assert 0 <= parents[i] < i
                    # siblings distinct; the subtree of parents[i] is contiguous (pre-order)
                    sib = [j for j in range(1, n) if parents[j] == parents[i] and j != i]
                    assert all(tokens[j] != tokens[i] for j in sib)
                    assert all(parents[j] >= parents[i] for j in range(parents[i] + 1, i))
                    assert q[i] <= q[parents[i]]
                # admission order is best first and every prefix is ancestor-closed
                keys = [_key_of(parents, tokens, q, i) for i in order]
                assert keys == sorted(keys)
                seen = {0}
                for i in order:
                    assert parents[i] in seen
                    seen.add(i)
                if V and nodes == 31:
                    # the whole tree is kept (at most 6 votes x depth 4 nodes): the
                    # root's children carry every vote, each vote having a next token
                    kids = [i for i in range(1, n) if parents[i] == 0]
                    assert abs(sum(q[i] for i in kids) - 1.0) < 1e-6
