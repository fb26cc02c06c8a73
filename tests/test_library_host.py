"""Host-side checks of the C-ABI library (no GPU calls)."""
import itertools
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "treeverify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    import greedy_draft_tree_amd as g
    lib = g.load_library()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(g.binding.SYMBOLS)


def test_host_accept_walk_matches_oracle_on_all_tiny_trees():
    import greedy_draft_tree_amd as g
    count = 0
    for n in range(1, 6):
        for rest in itertools.product(*[range(i) for i in range(1, n)]):
            parents = [-1] + list(rest)
            kids = {}
            for i in range(1, n):
                kids.setdefault(parents[i], []).append(i)
            for tok in itertools.product(range(3), repeat=n - 1):
                tokens = [7] + list(tok)
                if any(len({tokens[c] for c in cs}) != len(cs) for cs in kids.values()):
                    continue
                rng = np.random.default_rng(count)
                am = rng.integers(0, 3, n)
                assert g.accept_walk(parents, tokens, am) == oracle.accept_walk(parents, tokens, am)
                count += 1
    assert count > 500


def test_host_accept_walk_rejects_bad_trees():
    import greedy_draft_tree_amd as g
    for parents in ([0, 0], [-1, 1], [-1, 0, 3], list(range(-1, 32))):
        with pytest.raises(g.TVError):
            g.accept_walk(parents, [1] * len(parents), [1] * len(parents))
