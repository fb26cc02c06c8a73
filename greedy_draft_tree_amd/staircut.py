"""StairCut pieces on the host ("Drafters and tree verify", StairCut).

* ``cut``: the native cut (``tv_staircut``) of a candidate tree to the node
  count that maximises expected committed tokens per millisecond.
* ``PriceModel``: verify prices by context class, kind (chain or tree) and row
  count, in the pages' price-file format
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
    """Verify prices in ms by (context class, kind, rows); see the module doc."""

    def __init__(self, table: Optional[dict] = None, ema: float = 0.1):
        self.table = table or {}
        self.ema = ema
        self.step_ms = self.table.get("step_ms")
        self.file: Dict[int, Dict[str, Dict[int, float]]] = {}
        for key, kinds in self.table.items():
            if not str(key).lstrip("-").isdigit() or not isinstance(kinds, dict):
                continue
            self.file[int(key)] = {k: {int(r): float(ms) for r, ms in v.items()} for k, v in kinds.items()}
        self.live: Dict[Tuple[int, str], Dict[int, float]] = {}

    @classmethod
    def load(cls, path: str, ema: float = 0.1) -> "PriceModel":
        with open(path) as f:
            return cls(json.load(f), ema)

    def class_of(self, ctx: int) -> Optional[int]:
        if not self.file:
            return None
        lower = [c for c in self.file if c <= ctx]
        return max(lower) if lower else min(self.file)

    def _file_price(self, cls: Optional[int], kind: str, rows: int) -> float:
        if cls is None or kind not in self.file[cls] or not self.file[cls][kind]:
            return 1.0
        pts = sorted(self.file[cls][kind].items())
        rs = [r for r, _ in pts]
        ps = [p for _, p in pts]
        if rows <= rs[0]:
            return ps[0]
        if rows <= rs[-1]:
            return float(np.interp(rows, rs, ps))
        if self.step_ms is not None:
            step = float(self.step_ms)
        elif len(rs) >= 2:
            step = (ps[-1] - ps[-2]) / (rs[-1] - rs[-2])
        else:
            step = 0.0
        return ps[-1] + step * (rows - rs[-1])

    def prices(self, ctx: int, kind: str) -> np.ndarray:
        """Prices for rows 0..32 (index 0 unused), non-decreasing in rows."""
        cls = self.class_of(ctx)
        live = self.live.get((cls, kind), {})
        base = np.array([self._file_price(cls, kind, r) for r in range(TV_MAX_NODES + 1)])
        offs = [ms - base[r] for r, ms in live.items()]
        shift = float(np.mean(offs)) if offs else 0.0
        out = base + shift
        for r, ms in live.items():
            out[r] = ms
        out[0] = out[1]
        return np.maximum.accumulate(out)

    def price(self, ctx: int, kind: str, rows: int) -> float:
        return float(self.prices(ctx, kind)[rows])

    def observe(self, ctx: int, kind: str, rows: int, ms: float) -> None:
        """Follow a live price: an EMA of the counts seen (started at the
        model's current price for that count)."""
        cls = self.class_of(ctx)
        live = self.live.setdefault((cls, kind), {})
        cur = live.get(rows, self.price(ctx, kind, rows))
        live[rows] = cur + self.ema * (ms - cur)


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
