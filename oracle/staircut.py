"""StairCut, written plainly (TEST INFRASTRUCTURE: only tests may import it).

"Drafters and tree verify", StairCut: before each verify, the candidate
tree is trimmed to the size with the best ratio of expected tokens to cost,

    (1 + min(sum of q over the kept nodes, their number)) / (verify(rows) + draft + commit),

q being a node's path probability (the caller caps it at 1).  Candidates
enter in descending drafter score, and a node that enters brings along any
of its ancestors not yet kept; the sizes considered stop at 7, 15, 23 or 31
nodes (8, 16, 24 or 32 rows) and at the full candidate.

Readings taken here (the pages leave them open):
* a cut "ends at" P nodes means: the longest admission prefix whose kept set
  (the root excluded) has at most P nodes; the whole candidate is a cut when
  it has at most 31 nodes;
* rows = kept nodes + 1 (the root row, the last emitted token);
* the price uses the chain table when the kept nodes form one path from the
  root, else the tree table;
* among equal scores the smaller cut wins.
"""
from typing import List, Sequence, Tuple

STAIR_NODES = (7, 15, 23, 31)


def _with_ancestors(parents: Sequence[int], node: int) -> List[int]:
    out = []
    j = node
    while j >= 0:
        out.append(j)
        j = int(parents[j])
    return out


def is_chain(parents: Sequence[int], kept) -> bool:
    kids = {}
    for i in kept:
        if i != 0:
            kids[int(parents[i])] = kids.get(int(parents[i]), 0) + 1
    return all(c <= 1 for c in kids.values())


def staircut(parents: Sequence[int], q: Sequence[float], order: Sequence[int],
             price_tree: Sequence[float], price_chain: Sequence[float],
             draft_ms: float, commit_ms: float) -> Tuple[List[int], float]:
    """(kept node ids in increasing order, root first; the cut's score).
    price_*[rows] is the verify price in ms of `rows` rows (index 0 unused)."""
    kept = {0}
    prefixes = [frozenset(kept)]
    for node in order:
        kept |= set(_with_ancestors(parents, int(node)))
        prefixes.append(frozenset(kept))
    K = len(order)
    ends = set()
    for P in STAIR_NODES:
        ends.add(max(k for k in range(K + 1) if len(prefixes[k]) - 1 <= P))
    if len(prefixes[K]) - 1 <= STAIR_NODES[-1]:
        ends.add(K)
    best, best_k = None, None
    for k in sorted(ends, key=lambda k: (len(prefixes[k]), k)):
        s = prefixes[k]
        nodes = len(s) - 1
        qsum = 0.0
        for i in sorted(s):                        # node order
            if i != 0:
                qsum += float(q[i])
        gain = 1.0 + min(qsum, float(nodes))
        table = price_chain if is_chain(parents, s) else price_tree
        score = gain / (float(table[nodes + 1]) + draft_ms + commit_ms)
        if best is None or score > best:
            best, best_k = score, k
    return sorted(prefixes[best_k]), best
