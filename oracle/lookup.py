"""The lookup drafter over the request's own text, written plainly
(TEST INFRASTRUCTURE: only tests may import it).

"Drafters and tree verify", The lookup drafter: this drafter proposes
tokens by reuse, not by a model.  The request's most recent tokens (a suffix
of 2 to 8 ids) are searched for earlier in its own prompt and output; each
earlier place where the longest such suffix occurs contributes the tokens
that followed it, and merging those continuations gives a tree in which a
node's score is the fraction of continuations that pass through it.
StairCut then takes the tree, using that fraction as the node's q
("Drafters and tree verify", StairCut).

Readings taken here (the pages leave them open):
* an occurrence of order o is a start p with text[p:p+o] equal to the last o
  tokens and p + o <= len - 1: it ends before the text does, so it is
  followed by at least one token and is not the suffix itself;
* the order used is the largest o in [min_order, max_order] that has an
  occurrence; every occurrence of that order is one vote, and its
  continuation is text[p+o : p+o+max_depth] (shorter where the text ends);
* a node of the tree is a token sequence that begins at least one
  continuation; its count is the number of such continuations and its score
  q = count / votes, the share of votes through it (a path probability: the
  product of the conditional shares along the path);
* at most max_nodes nodes are kept, best first by (count descending, depth
  ascending, path ascending as a token sequence); an ancestor always comes
  before its descendants in that order, so every kept set is a tree;
* output: node 0 is the root, the text's last token (the next verify's
  root), q = 1; then the kept nodes in depth-first pre-order with siblings by
  (count descending, token ascending); ``order`` lists the kept nodes by
  admission (the best-first order above) as output indices;
* ``rho`` is the continuation rate a level that StairCut's q multiplies in
  ("Drafters and tree verify", StairCut: a fixed decay of 1/1.6 a level, or a
  learned rate that lets a long verbatim copy keep its whole line): a node at
  depth d gets q = (count / votes) * rho^d, rho^d taken as d products in fp64,
  rounded once to fp32; rho = 1 gives the plain vote shares.
"""
from typing import Dict, List, Sequence, Tuple


def match_order(text: Sequence[int], min_order: int, max_order: int) -> Tuple[int, List[int]]:
    """(o, starts): the largest order in [min_order, max_order] with an
    occurrence that ends before the text does, and the starts of all its
    occurrences in increasing order; (0, []) when there is none."""
    L = len(text)
    for o in range(max_order, min_order - 1, -1):
        if o > L - 1:
            continue
        suffix = list(text[L - o:])
        starts = [p for p in range(0, L - o) if list(text[p:p + o]) == suffix]
        if starts:
            return o, starts
    return 0, []


def node_counts(text: Sequence[int], starts: Sequence[int], o: int, max_depth: int) -> Dict[tuple, int]:
    """Count of every token sequence that begins a continuation."""
    counts: Dict[tuple, int] = {}
    for p in starts:
        cont = tuple(int(t) for t in text[p + o:p + o + max_depth])
        for d in range(1, len(cont) + 1):
            counts[cont[:d]] = counts.get(cont[:d], 0) + 1
    return counts


def lookup_draft(text: Sequence[int], min_order: int = 2, max_order: int = 8, max_depth: int = 31,
                 max_nodes: int = 31, rho: float = 1.0):
    """(parents, tokens, q, order, o, votes) of the lookup tree; q as fp32
    values (count / votes * rho^depth in fp64, rounded once)."""
    import numpy as np
    text = [int(t) for t in text]
    o, starts = match_order(text, min_order, max_order)
    root = text[-1]
    if not starts or max_nodes == 0:
        return [-1], [root], [1.0], [], o, len(starts)
    counts = node_counts(text, starts, o, max_depth)
    ranked = sorted(counts, key=lambda path: (-counts[path], len(path), path))
    kept = ranked[:max_nodes]
    keptset = set(kept)
    assert all(path[:-1] in keptset or len(path) == 1 for path in kept)
    # depth-first pre-order, siblings by (count desc, token asc)
    children: Dict[tuple, List[tuple]] = {(): []}
    for path in kept:
        children.setdefault(path, [])
        children.setdefault(path[:-1], []).append(path)
    for k in children:
        children[k].sort(key=lambda path: (-counts[path], path[-1]))
    parents, tokens, q, index = [-1], [root], [1.0], {(): 0}
    V = len(starts)

    def visit(path):
        for ch in children[path]:
            index[ch] = len(tokens)
            parents.append(index[path])
            tokens.append(ch[-1])
            decay = 1.0
            for _ in range(len(ch)):
                decay *= float(np.float32(rho))
            q.append(float(np.float32(counts[ch] / V * decay)))
            visit(ch)

    visit(())
    order = [index[path] for path in kept]
    return parents, tokens, q, order, o, V
