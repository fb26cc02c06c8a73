"""The native lookup drafter (tv_lookup_draft) against the oracle ("Drafters
and tree verify", The lookup drafter).  Host only: no GPU.

Bar: bit-exact (parents, tokens, q as fp32, admission order, order used,
votes) on seeded texts over small and large alphabets, short and long, with
repeats planted the way the pages' copy workloads make them (a quoted span
repeated later in the request), and at the edges (one token, no match,
max_nodes 0, every order bound).
"""
import numpy as np
import pytest

import synth
from oracle.lookup import lookup_draft as oracle_draft
from greedy_draft_tree_amd import TVError
from greedy_draft_tree_amd.lookup import draft
from greedy_draft_tree_amd.staircut import cut


def _same(text, *prm):
    got = draft(text, *prm)
    want = oracle_draft(text, *prm)
    assert tuple(got) == want, (list(text)[:20], prm)
    return got


def _quoted(rng, L, vocab):
    """Uniform ids with spans of the text copied further on (a quotation or an
    edit of text already in the context)."""
    t = [int(x) for x in rng.integers(0, vocab, L)]
    for _ in range(int(rng.integers(1, 6))):
        n = int(rng.integers(4, 40))
        a = int(rng.integers(0, max(1, L - n)))
        b = int(rng.integers(a, L))
        t[b:b + n] = t[a:a + n][:max(0, L - b)]
    return t


def test_random_texts_bit_exact():
    rng = np.random.default_rng(3)
    for i in range(400):
        L = int(rng.integers(1, 300))
        vocab = int(rng.choice([2, 3, 5, 50, 151936]))
        text = _quoted(rng, L, vocab) if i % 2 else [int(x) for x in rng.integers(0, vocab, L)]
        mn = int(rng.integers(1, 4))
        mx = int(rng.integers(mn, 12))
        rho = 1.0 if i % 3 else float(rng.choice([1 / 1.6, 0.9, 0.3]))
        _same(text, mn, mx, int(rng.integers(1, 40)), int(rng.integers(0, 64)), rho)


def test_long_texts_bit_exact():
    rng = np.random.default_rng(4)
    for L, vocab in ((4096, 151936), (5000, 7), (8192, 3)):
        text = _quoted(rng, L, vocab)
        for nodes in (31, 255):
            _same(text, 2, 8, 31, nodes)
            _same(text, 2, 8, 31, nodes, 1 / 1.6)


def test_edges():
    assert tuple(draft([7], 2, 8, 31, 31)) == ([-1], [7], [1.0], [], 0, 0)
    _same([7], 1, 1, 1, 0)
    _same([1, 1], 1, 8, 31, 31)
    _same([1, 1, 1, 1, 1, 1, 1, 1, 1, 1], 2, 8, 31, 0)
    _same([1] * 300, 2, 64, 256, 255)          # every bound at its maximum
    _same(list(range(50)) * 3, 8, 8, 1, 5)      # depth 1: a bush under the root
    # the pages' orders: a quoted line is copied whole
    line = synth.uniform_ids(40, 151936, 9).tolist()
    text = synth.uniform_ids(100, 151936, 10).tolist() + line + synth.uniform_ids(50, 151936, 11).tolist() + line[:12]
    t = _same(text, 2, 8, 31, 31)
    assert t.match_order == 8 and t.votes == 1
    assert len(t.tokens) == 32 and t.tokens[1:29] == line[12:] and t.q[1:] == [1.0] * 31


@pytest.mark.parametrize("args", [
    ([], 2, 8, 31, 31), ([1, 2], 0, 8, 31, 31), ([1, 2], 3, 2, 31, 31), ([1, 2], 2, 65, 31, 31),
    ([1, 2], 2, 8, 0, 31), ([1, 2], 2, 8, 257, 31), ([1, 2], 2, 8, 31, 256), ([1, 2], 2, 8, 31, -1)])
def test_invalid_arguments(args):
    with pytest.raises(TVError):
        draft(*args)


def test_native_rejects_bad_pointers_and_sizes():
    import ctypes
    from greedy_draft_tree_amd.binding import load_library
    lib = load_library()
    t = np.array([1, 2, 1, 2], np.int32)
    out = np.zeros(40, np.int32)
    qf = np.zeros(40, np.float32)
    n = ctypes.c_int(0)
    addr = lambda a: a.__array_interface__["data"][0]
    assert lib.tv_lookup_draft(None, 4, 2, 8, 31, 31, 1.0, addr(out), addr(out), addr(qf), addr(out), ctypes.byref(n),
                               None, None) == -1
    assert lib.tv_lookup_draft(addr(t), 0, 2, 8, 31, 31, 1.0, addr(out), addr(out), addr(qf), addr(out), ctypes.byref(n),
                               None, None) == -1
    assert lib.tv_lookup_draft(addr(t), 4, 2, 8, 31, 5, 1.0, addr(out), addr(out), addr(qf), None, ctypes.byref(n),
                               None, None) == -1
    assert lib.tv_lookup_draft(addr(t), 4, 2, 8, 31, 0, 1.0, addr(out), addr(out), addr(qf), None, ctypes.byref(n),
                               None, None) == 0 and n.value == 1
    for rho in (0.0, -0.5, 1.5, float("nan")):
        assert lib.tv_lookup_draft(addr(t), 4, 2, 8, 31, 5, rho, addr(out), addr(out), addr(qf), addr(out),
                                   ctypes.byref(n), None, None) == -1


def test_lookup_tree_feeds_staircut():
    """The drafter's q and admission order go straight into the cut; a copied
    line (one vote, q = 1 down the chain) is kept whole when verify prices are
    flat, and cut back when long verifies cost more than they return."""
    line = synth.uniform_ids(40, 151936, 12).tolist()
    text = synth.uniform_ids(60, 151936, 13).tolist() + line + line[:10]
    t = draft(text, 2, 8, 31, 31)
    assert t.votes == 1 and t.parents == [-1] + list(range(31))
    assert t.tokens[1:31] == line[10:] and t.tokens[31] == line[0]
    flat = [0.0] + [10.0] * 32
    keep, score = cut(t.parents, t.q, t.order, flat, flat, 1.0, 0.5)
    assert keep == list(range(32))
    steep = [0.0] + [10.0 + (40.0 if r > 8 else 0.0) for r in range(1, 33)]
    keep2, _ = cut(t.parents, t.q, t.order, steep, steep, 1.0, 0.5)
    assert keep2 == list(range(8))


def test_decay_keeps_or_cuts_a_copied_line():
    """StairCut on the MI355X price shape (a verify costs little more at 32
    rows than at 8): with the fixed decay of 1/1.6 a level a copied line is cut
    back, with a continuation rate of 1 it is kept whole, as the pages say of
    their learned rate for long verbatim copies."""
    from greedy_draft_tree_amd.lookup import STAIR_DECAY
    line = synth.uniform_ids(40, 151936, 14).tolist()
    text = synth.uniform_ids(60, 151936, 15).tolist() + line + line[:10]
    prices = [0.0] + [10.0 + 0.03 * r for r in range(1, 33)]
    whole = draft(text, 2, 8, 31, 31)
    decayed = draft(text, 2, 8, 31, 31, STAIR_DECAY)
    assert decayed.parents == whole.parents and decayed.order == whole.order
    for d in range(1, 32):
        r = 1.0
        for _ in range(d):
            r *= float(np.float32(STAIR_DECAY))
        assert decayed.q[d] == float(np.float32(r))
    keep, _ = cut(whole.parents, whole.q, whole.order, prices, prices, 1.0, 0.5)
    assert len(keep) == 32
    # decayed: sum q = (1 - 0.625^n) / 0.6 for n nodes; at 7 / 15 / 31 nodes the
    # score is 2.6043 / 11.74, 2.6652 / 11.98, 2.6667 / 12.46 ms: 15 nodes win
    keep, _ = cut(decayed.parents, decayed.q, decayed.order, prices, prices, 1.0, 0.5)
    assert len(keep) == 16
