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


class Prices:
    """Verify prices by row count, plainly ("Drafters and tree verify",
    StairCut on Flash-Next, and the shared price files): a price file lists
    prices by context class and kind (chain or tree); a context without its
    own class takes the nearest lower one; counts between two listed ones
    interpolate; past the last listed count the price grows step_ms a row,
    or by the last two counts' slope; measured rounds update a count's price
    online (an EMA of weight `ema` a count) and shift the counts not measured
    by the learned offset; a price never falls with more rows; with no file
    every count costs 1 ms.

    Readings taken here: a context below every listed class takes the
    smallest one; a count below the first listed one takes the first listed
    price; the learned offset is the mean of (live price - file price) over
    the measured counts of that class and kind; a count's live price starts
    at its current price; the table is made non-decreasing by a running
    maximum from one row upward, and row 0 copies row 1.

    points: (context class, kind, rows, ms) tuples, kind "chain" or "tree".
    """

    ROWS = 32

    def __init__(self, points, step_ms=None, ema=0.1):
        self.curves = {}
        for c, k, r, m in points:
            self.curves.setdefault((c, k), {})[r] = m
        self.classes = sorted({c for c, _, _, _ in points})
        self.step_ms = step_ms
        self.ema = ema
        self.live = {}   # (class, kind) -> {rows: ms}, in the order first measured

    def context_class(self, ctx):
        if not self.classes:
            return None
        lower = [c for c in self.classes if c <= ctx]
        return max(lower) if lower else self.classes[0]

    def file_price(self, cls, kind, rows):
        pts = sorted(self.curves.get((cls, kind), {}).items())
        if cls is None or not pts:
            return 1.0
        if rows <= pts[0][0]:
            return pts[0][1]
        for (r0, p0), (r1, p1) in zip(pts, pts[1:]):
            if r0 <= rows <= r1:
                return p0 + (p1 - p0) * (rows - r0) / (r1 - r0)
        r_last, p_last = pts[-1]
        if self.step_ms is not None:
            step = self.step_ms
        elif len(pts) >= 2:
            step = (p_last - pts[-2][1]) / (r_last - pts[-2][0])
        else:
            step = 0.0
        return p_last + step * (rows - r_last)

    def table(self, ctx, kind):
        cls = self.context_class(ctx)
        base = [self.file_price(cls, kind, r) for r in range(self.ROWS + 1)]
        live = self.live.get((cls, kind), {})
        shift = sum(ms - base[r] for r, ms in live.items()) / len(live) if live else 0.0
        out = [b + shift for b in base]
        for r, ms in live.items():
            out[r] = ms
        out[0] = out[1]
        for r in range(1, self.ROWS + 1):
            out[r] = max(out[r], out[r - 1])
        return out

    def observe(self, ctx, kind, rows, ms):
        cls = self.context_class(ctx)
        live = self.live.setdefault((cls, kind), {})
        cur = live[rows] if rows in live else self.table(ctx, kind)[rows]
        live[rows] = cur + self.ema * (ms - cur)
