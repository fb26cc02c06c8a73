"""StairCut pieces on the host ("Drafters and tree verify", StairCut).

* ``cut``: the native cut (``tv_staircut``) of a candidate tree to the node
  count that maximises expected committed tokens per millisecond.
* ``PriceModel``: the library's verify prices (``tv_prices_*``) by context
  class, kind (chain or tree) and row count, from a price file in the pages'
  format
  ``{"<context class>": {"<kind>": {"<rows>": ms, ...}, ...}, ..., "step_ms": x, "measured": "..."}``,
  and the rules the pages give for reading it ("Drafters and tree verify",
  StairCut on Flash-Next, and the shared price files): an unlisted context
  class falls back to the largest listed one below it; a row count between
  two measured ones is a linear blend of them; beyond the last measured
  count the price grows by ``step_ms`` per row, or by the slope of the last
  two counts when the file has no ``step_ms``; measured round times update
  the prices online with an exponential moving average of weight 0.1 per
  count, shifting the unmeasured counts by the mean learned offset; prices
  are made non-decreasing in the row count.  With no file, every count
  costs 1 ms.
* ``measure_prices``: a price file for a bound model on this GPU.
"""
from __future__ import annotations

import ctypes
import json
import time
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .binding import TV_MAX_NODES, TV_MAX_CANDIDATE, TVError, _i32, _ptr, load_library

KINDS = ("chain", "tree")


def cut(parents: Sequence[int], q: Sequence[float], order: Sequence[int], price_tree: Sequence[float],
        price_chain: Sequence[float], draft_ms: float, commit_ms: float) -> Tuple[List[int], float]:
    """tv_staircut: (kept node ids, root first; the cut's tokens per ms).
    price_*[rows] in ms for rows 1..32 (index 0 unused)."""
    lib = load_library()
    p, o = _i32(parents), _i32(order)
    n = len(p)
    if n < 1 or n > TV_MAX_CANDIDATE or len(o) != n - 1:
        raise TVError(-1, "tv_staircut: bad candidate size")
    qa = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    pt = np.ascontiguousarray(np.asarray(price_tree, dtype=np.float32))
    pc = np.ascontiguousarray(np.asarray(price_chain, dtype=np.float32))
    if pt.shape[0] < TV_MAX_NODES + 1 or pc.shape[0] < TV_MAX_NODES + 1 or qa.shape[0] < n:
        raise TVError(-1, "tv_staircut: price tables need rows 1..32")
    keep = np.zeros(TV_MAX_NODES, np.int32)
    nk = ctypes.c_int(0)
    score = ctypes.c_float(0.0)
    rc = lib.tv_staircut(_ptr(p), _ptr(qa), _ptr(o) if n > 1 else None, n, _ptr(pt), _ptr(pc),
                         float(draft_ms), float(commit_ms), _ptr(keep), ctypes.byref(nk), ctypes.byref(score))
    if rc != 0:
        raise TVError(rc, "tv_staircut: invalid candidate or prices")
    return keep[:nk.value].tolist(), float(score.value)


class PriceModel:
    """Verify prices in ms by (context class, kind, rows): the library's
    price model (``tv_prices_*``) built from a price file in the format of
    the module doc; this class only marshals."""

    def __init__(self, table: Optional[dict] = None, ema: float = 0.1):
        self.table = table or {}
        self.ema = ema
        step = self.table.get("step_ms")
        cls, kind, rows, ms = [], [], [], []
        for key, kinds in self.table.items():
            if not str(key).lstrip("-").isdigit() or not isinstance(kinds, dict):
                continue
            for k, v in kinds.items():
                if k not in KINDS:
                    continue
                for r, p in v.items():
                    cls.append(int(key))
                    kind.append(KINDS.index(k))
                    rows.append(int(r))
                    ms.append(float(p))
        self._lib = load_library()
        c, kd, rw = _i32(cls), _i32(kind), _i32(rows)
        m = np.ascontiguousarray(np.asarray(ms, dtype=np.float64))
        h = ctypes.c_void_p()
        rc = self._lib.tv_prices_create(_ptr(c) if len(cls) else None, _ptr(kd) if len(cls) else None,
                                        _ptr(rw) if len(cls) else None, _ptr(m) if len(cls) else None, len(cls),
                                        int(step is not None), float(step) if step is not None else 0.0,
                                        float(ema), ctypes.byref(h))
        if rc != 0:
            raise TVError(rc, "tv_prices_create: invalid price file or weight")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.tv_prices_destroy(h)
            self._h = None

    @classmethod
    def load(cls, path: str, ema: float = 0.1) -> "PriceModel":
        with open(path) as f:
            return cls(json.load(f), ema)

    def class_of(self, ctx: int) -> Optional[int]:
        c, has = ctypes.c_int32(0), ctypes.c_int(0)
        rc = self._lib.tv_prices_class(self._h, int(ctx), ctypes.byref(c), ctypes.byref(has))
        if rc != 0:
            raise TVError(rc, "tv_prices_class")
        return int(c.value) if has.value else None

    def prices(self, ctx: int, kind: str) -> np.ndarray:
        """Prices for rows 0..32 (index 0 unused), non-decreasing in rows."""
        out = np.zeros(TV_MAX_NODES + 1, np.float64)
        rc = self._lib.tv_prices_table(self._h, int(ctx), KINDS.index(kind), _ptr(out))
        if rc != 0:
            raise TVError(rc, "tv_prices_table")
        return out

    def price(self, ctx: int, kind: str, rows: int) -> float:
        return float(self.prices(ctx, kind)[rows])

    def observe(self, ctx: int, kind: str, rows: int, ms: float) -> None:
        """Follow a live price: an EMA of the counts seen (started at the
        model's current price for that count)."""
        rc = self._lib.tv_prices_observe(self._h, int(ctx), KINDS.index(kind), int(rows), float(ms))
        if rc != 0:
            raise TVError(rc, "tv_prices_observe: bad kind, count or time")


def _tree_shape(rows: int, kind: str) -> List[int]:
    """A verify shape of `rows` rows: a chain, or a spine of about half the
    rows with the other nodes as leaves spread along it."""
    if kind == "chain" or rows <= 2:
        return [-1] + list(range(rows - 1))
    spine = (rows + 1) // 2
    parents = [-1] + list(range(spine - 1))
    for i in range(rows - spine):
        parents.append(i % spine)
    return parents


def measure_prices(tv, req: int, ctx_lens: Iterable[int], rows: Iterable[int] = range(1, TV_MAX_NODES + 1),
                   kinds: Sequence[str] = KINDS, reps: int = 5, warmup: int = 2, note: str = "") -> dict:
    """A price file for the model bound to ``tv``: the median wall time of
    ``reps`` verifies (host call to host results) per (context length, kind,
    rows).  The request's cache rows below each length must be bound; their
    contents do not matter for the price.  The request's context is left at
    the last length measured."""
    out: dict = {}
    rows = list(rows)
    for ctx in ctx_lens:
        tv.set_history(req, [], int(ctx))
        out[str(int(ctx))] = {}
        for kind in kinds:
            table = {}
            for r in rows:
                parents = _tree_shape(r, kind)
                tokens = [(i * 7919 + 17) % tv.vocab for i in range(r)]
                for _ in range(warmup):
                    tv.verify_tree(req, parents, tokens)
                ts = []
                for _ in range(reps):
                    t0 = time.perf_counter()
                    tv.verify_tree(req, parents, tokens)
                    ts.append((time.perf_counter() - t0) * 1e3)
                table[str(r)] = round(float(np.median(ts)), 4)
            out[str(int(ctx))][kind] = table
    slopes = []
    for ctx in out:
        for kind in out[ctx]:
            t = out[ctx][kind]
            if len(rows) >= 2:
                slopes.append((t[str(rows[-1])] - t[str(rows[-2])]) / (rows[-1] - rows[-2]))
    out["step_ms"] = round(float(max(0.0, np.median(slopes))) if slopes else 0.0, 4)
    out["measured"] = note or (f"median of {reps} verifies (host call to host results) per count, "
                               f"{time.strftime('%Y-%m-%d')}")
    return out
