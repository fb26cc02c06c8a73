"""The lookup drafter on the host ("Drafters and tree verify", The lookup
drafter): a draft tree copied from the request's own text.

``draft`` calls ``tv_lookup_draft``: the longest match (orders min..max) of
the text's last tokens among earlier occurrences, one vote per occurrence,
and the best ``max_nodes`` nodes of the votes' continuation tree with their
vote shares as q (times rho^depth: StairCut's continuation rate a level).  The result plugs into StairCut (``staircut.cut``): q and
the admission order are what it takes.
"""
from __future__ import annotations

import ctypes
from typing import List, NamedTuple, Sequence

import numpy as np

from .binding import TV_LOOKUP_MAX_ORDER, TV_MAX_CANDIDATE, TVError, _i32, _ptr, load_library


class LookupTree(NamedTuple):
    parents: List[int]     # node 0 the root (the text's last token)
    tokens: List[int]
    q: List[float]         # vote shares (fp32 values), q[0] = 1
    order: List[int]       # kept nodes by admission, as indices
    match_order: int       # order of the match used (0: nothing matched)
    votes: int


STAIR_DECAY = 1.0 / 1.6   # StairCut's fixed continuation rate a level for lookup nodes


def draft(text: Sequence[int], min_order: int = 2, max_order: int = 8, max_depth: int = 31,
          max_nodes: int = 31, rho: float = 1.0) -> LookupTree:
    """tv_lookup_draft.  q = vote share * rho^depth: rho = 1 gives the plain
    shares, STAIR_DECAY the q StairCut takes with its fixed decay."""
    lib = load_library()
    t = _i32(text)
    if t.ndim != 1 or t.shape[0] < 1:
        raise TVError(-1, "tv_lookup_draft: the text needs at least one token")
    if not (0 <= max_nodes < TV_MAX_CANDIDATE) or not (1 <= min_order <= max_order <= TV_LOOKUP_MAX_ORDER):
        raise TVError(-1, "tv_lookup_draft: bad orders or node count")
    cap = max_nodes + 1
    parents = np.empty(cap, np.int32)
    tokens = np.empty(cap, np.int32)
    q = np.empty(cap, np.float32)
    order = np.empty(max(max_nodes, 1), np.int32)
    n, o, v = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    if not (0.0 < rho <= 1.0):
        raise TVError(-1, "tv_lookup_draft: rho must lie in (0, 1]")
    rc = lib.tv_lookup_draft(_ptr(t), int(t.shape[0]), min_order, max_order, max_depth, max_nodes, rho,
                             _ptr(parents), _ptr(tokens), _ptr(q), _ptr(order),
                             ctypes.byref(n), ctypes.byref(o), ctypes.byref(v))
    if rc != 0:
        raise TVError(rc, "tv_lookup_draft: invalid arguments")
    k = n.value
    return LookupTree(parents[:k].tolist(), tokens[:k].tolist(), [float(x) for x in q[:k]],
                      order[:k - 1].tolist(), o.value, v.value)
