"""Seeded synthetic inputs for the tree-verify path.

This module is test and benchmark infrastructure shared by the CPU oracle and
the HIP library's callers.  It draws random numbers and lays out shapes; it
holds none of the method's arithmetic (no norm, projection, attention, walk or
commit).  Everything is a pure function of its seed.

Recipe (also the workload stand-in for the pages' private prompt sets):

* weights: every matrix, the embedding and the output head are N(0, 0.02)
  drawn in fp32 by torch's generator on the named device and rounded to bf16;
  norm weights are 1 (bf16).  Tensor ``i`` of a model is drawn with seed
  ``seed * 1_000_003 + i``.  The CPU and CUDA generators give different draws
  for one seed, so a weight set is named by (seed, device).
* synthetic KV cache: N(0, 1) rows, bf16, taken to be already rotated.
* recurrent start state: N(0, 1) fp32 per head.
* token ids (prompts, histories, draft tokens): uniform over the vocabulary.
* trees: a spine with single-token branches, DFS pre-order (``spine_tree``).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# Layer kinds.
ATTN = 0
RECUR = 1    # gated linear recurrence
DELTA = 2    # gated delta rule


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shapes of a decoder-only target model (no arithmetic here)."""

    name: str
    n_layer: int
    hidden: int
    n_qhead: int
    n_kvhead: int
    head_dim: int
    ffn: int
    vocab: int
    kinds: Tuple[int, ...]  # per layer: ATTN, RECUR or DELTA
    eps: float = 1e-6
    rope_theta: float = 1e4

    @property
    def qkv_rows(self) -> int:
        return (self.n_qhead + 2 * self.n_kvhead) * self.head_dim

    @property
    def rqkv_rows(self) -> int:
        return 3 * self.n_qhead * self.head_dim


def _shape(name, n_layer, hidden, qh, kvh, d, ffn, vocab, kinds=None):
    if kinds is None:
        kinds = tuple([ATTN] * n_layer)
    return ModelShape(name, n_layer, hidden, qh, kvh, d, ffn, vocab, tuple(kinds))


# The five workloads.  c2 is 64 copies of the c1 layer; c3 makes layer l
# recurrent unless l % 4 == 3 (48 recurrent + 16 attention layers).
C0 = _shape("c0_tiny", 2, 256, 4, 2, 64, 688, 1024)
C1 = _shape("c1_layer", 1, 5120, 40, 8, 128, 17408, 151936)
C2 = _shape("c2_stack64", 64, 5120, 40, 8, 128, 17408, 151936)
C3 = _shape("c3_hybrid64", 64, 5120, 40, 8, 128, 17408, 151936,
            kinds=[RECUR if (l % 4) != 3 else ATTN for l in range(64)])
# c3 with gated delta-rule layers in place of the plain gated recurrence: the
# pages' 48 Gated DeltaNet + 16 attention layers
C3D = _shape("c3d_delta64", 64, 5120, 40, 8, 128, 17408, 151936,
             kinds=[DELTA if (l % 4) != 3 else ATTN for l in range(64)])

SHAPES = {s.name: s for s in (C0, C1, C2, C3, C3D)}


def scaled(shape: ModelShape, name: str, n_layer: Optional[int] = None,
           kinds: Optional[Sequence[int]] = None, **kw) -> ModelShape:
    """A variant of ``shape`` (used by tests for mid-size cases)."""
    d = dataclasses.asdict(shape)
    d["name"] = name
    if n_layer is not None:
        d["n_layer"] = n_layer
        if kinds is None:
            kinds = [shape.kinds[l % len(shape.kinds)] for l in range(n_layer)]
    if kinds is not None:
        d["kinds"] = tuple(kinds)
    d.update(kw)
    return ModelShape(**d)


def weight_names(shape: ModelShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, kind) of every tensor; kind is 'normal' or 'ones'."""
    H, V = shape.hidden, shape.vocab
    QD = shape.n_qhead * shape.head_dim
    out = [("emb", (V, H), "normal")]
    for l, k in enumerate(shape.kinds):
        p = f"layers.{l}."
        out.append((p + "attn_norm", (H,), "ones"))
        if k == ATTN:
            out.append((p + "wqkv", (shape.qkv_rows, H), "normal"))
        else:
            out.append((p + "wqkv", (shape.rqkv_rows, H), "normal"))
            # gate rows; a delta layer stacks its write-strength rows under them
            rows = shape.n_qhead if k == RECUR else 2 * shape.n_qhead
            out.append((p + "wa", (rows, H), "normal"))
        out.append((p + "wo", (H, QD), "normal"))
        out.append((p + "ffn_norm", (H,), "ones"))
        out.append((p + "wg", (shape.ffn, H), "normal"))
        out.append((p + "wu", (shape.ffn, H), "normal"))
        out.append((p + "wd", (H, shape.ffn), "normal"))
    out.append(("final_norm", (H,), "ones"))
    out.append(("head", (V, H), "normal"))
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal_bf16(shape, seed, std, device, out: Optional[torch.Tensor] = None):
    """N(0, std) drawn in fp32 and rounded to bf16; chunked over rows."""
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    g = _gen(seed, device)
    rows = shape[0]
    per = max(1, (1 << 26) // max(1, int(np.prod(shape[1:])) if len(shape) > 1 else 1))
    for r0 in range(0, rows, per):
        r1 = min(rows, r0 + per)
        t = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                        dtype=torch.float32, device=device)
        out[r0:r1] = (t * std).to(torch.bfloat16)
    return out


def weights(shape: ModelShape, seed: int = 0, device="cpu",
            only: Optional[Sequence[str]] = None) -> Dict[str, torch.Tensor]:
    """All weights of ``shape`` as bf16 tensors on ``device``."""
    out = {}
    for i, (name, shp, kind) in enumerate(weight_names(shape)):
        if only is not None and name not in only:
            continue
        if kind == "ones":
            out[name] = torch.ones(shp, dtype=torch.bfloat16, device=device)
        else:
            out[name] = _normal_bf16(shp, seed * 1_000_003 + i, 0.02, device)
    return out


def uniform_ids(n: int, vocab: int, seed: int) -> np.ndarray:
    g = _gen(seed, "cpu")
    return torch.randint(0, vocab, (n,), generator=g, dtype=torch.int64).numpy().astype(np.int32)


def kv_cache(shape: ModelShape, ctx: int, seed: int, cap: Optional[int] = None,
             device="cpu", layers: Optional[Sequence[int]] = None):
    """Synthetic N(0,1) bf16 K and V per attention layer, [KVH, cap, D].

    Rows [0, ctx) hold the draw; rows beyond are zero.  Layer l's K uses seed
    ``seed*1_000_003 + 2l`` and its V ``+ 2l + 1``.
    """
    cap = ctx if cap is None else cap
    out = {}
    for l, k in enumerate(shape.kinds):
        if k != ATTN or (layers is not None and l not in layers):
            continue
        for j, nm in enumerate(("k", "v")):
            t = torch.zeros((shape.n_kvhead, cap, shape.head_dim), dtype=torch.bfloat16, device=device)
            if ctx > 0:
                src = _normal_bf16((shape.n_kvhead, ctx, shape.head_dim),
                                   seed * 1_000_003 + 2 * l + j, 1.0, device)
                t[:, :ctx] = src
            out[(l, nm)] = t
    return out


def state0(shape: ModelShape, seed: int, device="cpu", layers: Optional[Sequence[int]] = None):
    """Synthetic N(0,1) fp32 start state [QH, D, D] per recurrent layer."""
    out = {}
    for l, k in enumerate(shape.kinds):
        if k == ATTN or (layers is not None and l not in layers):
            continue
        g = _gen(seed * 1_000_003 + l, device)
        out[l] = torch.randn((shape.n_qhead, shape.head_dim, shape.head_dim),
                             generator=g, dtype=torch.float32, device=device)
    return out


# ---------------------------------------------------------------- trees

def spine_tree(n: int, seed: int, max_extra: int = 3, max_spine: int = 15) -> np.ndarray:
    """Parents (DFS pre-order) of an n-node tree: a spine plus single leaves.

    Spine depth ``D = min(max_spine, ceil((n-1)/2))``; the other ``n-1-D``
    nodes are leaves hung under seeded spine nodes 0..D-1, at most
    ``max_extra`` extra children per spine node.  In pre-order, each spine
    node's spine child comes first, then its leaves.
    """
    if n < 1:
        raise ValueError("n >= 1")
    D = min(max_spine, math.ceil((n - 1) / 2))
    B = n - 1 - D
    rng = np.random.default_rng(seed)
    leaves = [0] * max(D, 1)
    if B > max_extra * max(D, 1):
        raise ValueError("too many branches for the spine")
    placed = 0
    while placed < B:
        s = int(rng.integers(0, D))
        if leaves[s] < max_extra:
            leaves[s] += 1
            placed += 1
    parents: List[int] = []

    def visit(spine_idx: int, parent: int):
        me = len(parents)
        parents.append(parent)
        if spine_idx < D:
            visit(spine_idx + 1, me)
            for _ in range(leaves[spine_idx]):
                parents.append(me)

    visit(0, -1)
    assert len(parents) == n, (len(parents), n)
    return np.array(parents, dtype=np.int32)


def c0_tree() -> np.ndarray:
    """The tiny workload's 8-node tree: spine 0-1-2-3-4 with one leaf under
    each of nodes 2, 1 and 0, in DFS pre-order."""
    return np.array([-1, 0, 1, 2, 3, 2, 1, 0], dtype=np.int32)


def chain_tree(n: int) -> np.ndarray:
    return np.arange(-1, n - 1, dtype=np.int32)


def bush_tree(n: int) -> np.ndarray:
    """A root with n-1 leaf children."""
    p = np.zeros(n, dtype=np.int32)
    p[0] = -1
    return p


def random_tree(n: int, seed: int) -> np.ndarray:
    """A random recursive tree relabelled into DFS pre-order."""
    rng = np.random.default_rng(seed)
    par = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
    kids: List[List[int]] = [[] for _ in range(n)]
    for i in range(1, n):
        kids[par[i]].append(i)
    order: List[int] = []
    stack = [0]
    while stack:
        v = stack.pop()
        order.append(v)
        stack.extend(reversed(kids[v]))
    new = {old: i for i, old in enumerate(order)}
    out = np.empty(n, dtype=np.int32)
    for old in range(n):
        out[new[old]] = -1 if par[old] < 0 else new[par[old]]
    return out


def tree_tokens(parents: np.ndarray, vocab: int, seed: int, root_token: int,
                forced: Optional[Dict[int, int]] = None) -> np.ndarray:
    """Uniform draft tokens with distinct siblings (resample on collision).

    ``forced`` maps node index -> token to place (e.g. a drafter's spine);
    a forced token that collides with an earlier sibling is re-drawn.
    """
    rng = np.random.default_rng(seed)
    n = len(parents)
    tok = np.empty(n, dtype=np.int32)
    tok[0] = root_token
    seen: Dict[int, set] = {}
    for i in range(1, n):
        s = seen.setdefault(int(parents[i]), set())
        t = None if forced is None else forced.get(i)
        while t is None or t in s:
            t = int(rng.integers(0, vocab))
        s.add(t)
        tok[i] = t
    return tok


def spine_nodes(parents: np.ndarray) -> List[int]:
    """Indices of the spine: the root, then each node's first child."""
    n = len(parents)
    first_child = [-1] * n
    for i in range(n - 1, 0, -1):
        first_child[parents[i]] = i
    out = [0]
    while first_child[out[-1]] >= 0:
        out.append(first_child[out[-1]])
    return out


# ------------------------------------------------------------ modifiers

@dataclasses.dataclass
class Modifiers:
    rep_penalty: float
    bias_ids: np.ndarray   # int32 [n_bias], distinct
    bias_vals: np.ndarray  # float32 [n_bias]
    allow_bits: Optional[np.ndarray]  # uint32 [ceil(V/32)] or None


def modifiers(vocab: int, seed: int, n_bias: int = 64, bias: float = 5.0,
              penalty: float = 1.1, allow_frac: Optional[float] = 0.5) -> Modifiers:
    rng = np.random.default_rng(seed)
    ids = rng.choice(vocab, size=n_bias, replace=False).astype(np.int32)
    vals = np.where(rng.random(n_bias) < 0.5, -bias, bias).astype(np.float32)
    bits = None
    if allow_frac is not None:
        allow = rng.random(vocab) < allow_frac
        words = np.zeros((vocab + 31) // 32, dtype=np.uint32)
        idx = np.nonzero(allow)[0]
        np.bitwise_or.at(words, idx // 32, (np.uint32(1) << (idx % 32).astype(np.uint32)))
        bits = words
    return Modifiers(float(penalty), ids, vals, bits)


# ---------------------------------------------------- kernel-level inputs

def bf16_normal(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """N(0, std) drawn in fp32 and rounded to bf16 (one tensor)."""
    return _normal_bf16(tuple(shape), seed, std, device)


def dyadic_partials(splits: int, rows: int, cols: int, seed: int, std: float = 1.0) -> np.ndarray:
    """[splits, rows, cols] float32 split-K partials whose values are
    multiples of 2**-12 below 2**8 in magnitude, drawn around N(0, std/sqrt
    (splits)) per split: any order of fp32 additions of one element's
    partials is exact, so the sum has one value on every side."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, std / math.sqrt(splits), size=(splits, rows, cols))
    x = np.clip(np.round(x * 4096.0), -(2 ** 20 - 1), 2 ** 20 - 1) / 4096.0
    return x.astype(np.float32)


def splitk_layout(parts: np.ndarray) -> np.ndarray:
    """Lay [S, rows <= 32, cols] partials out in the library's split-K layout:
    column n of row m of k-range s at ((n // 128) * S + s) * 4096 + m * 128
    + n % 128 (a flat float32 array; unused places are zero)."""
    S, rows, cols = parts.shape
    assert rows <= 32
    nb = (cols + 127) // 128
    out = np.zeros((nb, S, 32, 128), dtype=np.float32)
    padded = np.zeros((S, rows, nb * 128), dtype=np.float32)
    padded[:, :, :cols] = parts
    out[:, :, :rows, :] = padded.reshape(S, rows, nb, 128).transpose(2, 0, 1, 3)
    return out.reshape(-1)
