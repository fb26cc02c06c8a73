"""CPU oracle for greedy tree verify.

TEST INFRASTRUCTURE.  This package is the slow, plain reference that the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it; the library
(``greedy_draft_tree_amd``) never does, and the two share no code.  The only
common module is ``synth`` (seeded inputs, no arithmetic of the method).

What it computes, and where the pages define it:

* ``Oracle.step``: one token through the target model, the "one forward pass
  per token" of plain greedy decoding ("Exactness", The promise).  The model
  is a pre-norm decoder; its arithmetic is fp64 with bf16 (round to nearest
  even) at the activation rounding points and an fp32 head output ("Exactness",
  The one exception: near ties: the head returns fp32 logits).  ``exact=True``
  drops every rounding point (used to pin the forward to an independent
  library implementation).
* ``Oracle.tree_scores``: the brute-force tree scorer.  Row i is the model's
  scores after consuming the path root..i, i.e. the sequential decode of the
  node's ancestor prefix ("Drafters and tree verify", The round, step 2;
  "Algorithm and correctness contract", Target position and batching, which
  indexes the same contexts by the child).
* ``apply_modifiers`` / ``top2``: score modifiers as plain decoding applies
  them to its one row ("Exactness", The promise; penalties before the other
  filters, "Exactness", Sampling), then argmax (lowest id on an exact tie)
  and the top-1/top-2 gap in bf16 ulps ("Exactness", The one exception).
* ``accept_walk``: the greedy accept walk with the bonus token ("Drafters and
  tree verify", The round, step 3).
* ``sample_keys`` / ``sampled_tree_decisions`` / ``sampled``: the sampled
  request.  The token at sequence index t is the argmax of the modified
  scores divided by the temperature plus Gumbel noise keyed by (seed, t)
  ("Exactness", Sampling; "Drafters and tree verify", Sampling); the noise
  comes from Philox4x32-10, written from its published definition.
* ``Seq.commit``: the oracle's committed state is its token sequence; a
  commit simply steps the accepted tokens one at a time ("Drafters and tree
  verify", The round, step 4).  The closed form of the recurrent state
  ("Drafters and tree verify", Tree verify through recurrent layers) is NOT
  used here; tests check it against this loop.
* Recurrent layers come in two kinds: a gated linear recurrence
  (``recur_mix``: S = e^g S_parent + k v^T) and the gated delta rule of the
  pages' Gated DeltaNet layers (``delta_mix``: S = e^g (I - beta k k^T)
  S_parent + beta k v^T, beta = sigmoid of a second projection), both
  stepped one token at a time.

Every pin that holds this code to the pages and to the mathematics lives in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from synth import ATTN, DELTA, RECUR, ModelShape, Modifiers

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_matvec.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C primitive with gcc (plain x86-64, OpenMP)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "matvec.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-o", tmp, src])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        lib.orc_matvec_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p]
        lib.orc_matvec_bf16.restype = None
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_get_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(_load().orc_get_threads())


# ------------------------------------------------------------ numerics

def bf16_round(x):
    """Round fp64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and binary32's exponent range, so a finite
    x is rounded on the grid of its quantum ``ulp_bf16(x)``.
    """
    x = np.asarray(x, dtype=np.float64)
    q = ulp_bf16(x)
    return np.rint(x / q) * q


def ulp_bf16(x):
    """One bf16 step at x: 2**(floor(log2|x|) - 7), or 2**-133 below the
    normal range (|x| < 2**-126, zero included)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)              # x = m * 2**e with m in [0.5, 1)
    e = np.where(x < 2.0 ** -126, -126, e - 1)
    return np.ldexp(1.0, e - 7)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of one row in fp64: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps) * np.asarray(w, dtype=np.float64)


def log_sigmoid(a):
    return -np.logaddexp(0.0, -np.asarray(a, dtype=np.float64))


def sigmoid(a):
    return np.exp(log_sigmoid(a))


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def t2u16(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor (CPU) -> uint16 numpy view of its bits."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def t2f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


# ------------------------------------------------------------ the model

class Oracle:
    """The target model of a ``synth.ModelShape`` on given bf16 weights.

    Weights are the spec's: every matrix is [N_out, K_in] row-major bf16;
    a layer's ``wqkv`` stacks q heads, then k heads, then v heads.
    """

    def __init__(self, shape: ModelShape, weights: Dict[str, torch.Tensor], exact: bool = False):
        self.s = shape
        self.exact = exact
        self.W = {k: t2u16(v) for k, v in weights.items()}
        for name, arr in self.W.items():
            assert arr.flags["C_CONTIGUOUS"], name
        self.lib = _load()
        D = shape.head_dim
        # RoPE frequencies, rotate-half pairing (i, i + D/2), fp64.
        self.inv_freq = shape.rope_theta ** (-(2.0 * np.arange(D // 2)) / D)

    # rounding point: bf16 unless exact
    def r(self, x):
        return np.asarray(x, dtype=np.float64) if self.exact else bf16_round(x)

    def matvec(self, name: str, x: np.ndarray) -> np.ndarray:
        W = self.W[name]
        N, K = W.shape
        x = np.ascontiguousarray(x, dtype=np.float64)
        assert x.shape == (K,)
        y = np.empty(N, dtype=np.float64)
        self.lib.orc_matvec_bf16(W.ctypes.data, N, K, x.ctypes.data, y.ctypes.data)
        return y

    def rmsnorm(self, x: np.ndarray, wname: str) -> np.ndarray:
        return rms_norm(x, bf16_bits_to_f64(self.W[wname]), self.s.eps)

    def rope(self, x: np.ndarray, pos: int) -> np.ndarray:
        """Rotate each head [h, D] by angle pos*inv_freq[i] on pairs (i, i+D/2)."""
        half = self.s.head_dim // 2
        ang = pos * self.inv_freq
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[:, :half], x[:, half:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=1)

    def attention(self, q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
        """q [QH, D]; K, V [KVH, L, D]; grouped heads; scaled dot product,
        softmax with max subtraction."""
        QH, D = q.shape
        grp = QH // K.shape[0]
        out = np.empty_like(q)
        for h in range(QH):
            kv = h // grp
            sc = K[kv] @ q[h] / math.sqrt(D)
            p = np.exp(sc - sc.max())
            out[h] = (p / p.sum()) @ V[kv]
        return out

    @staticmethod
    def recur_mix(q, k, v, g, S_prev):
        """Gated linear recurrence, one token, every head at once:
        S = exp(g) * S_prev + k v^T, read out o = S^T q.
        q, k, v [QH, D]; g [QH] (log of the decay); S [QH, D(k), D(v)]."""
        S = np.exp(g)[:, None, None] * S_prev + k[:, :, None] * v[:, None, :]
        o = np.einsum("hkv,hk->hv", S, q)
        return o, S

    @staticmethod
    def delta_mix(q, k, v, g, beta, S_prev):
        """Gated delta rule, one token, every head at once (Yang, Kautz and
        Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
        Rule", ICLR 2025): the state first decays by alpha = exp(g), then
        the value it returns for key k is moved a fraction beta of the way
        to v:  S = alpha (I - beta k k^T) S_prev + beta k v^T  (key index
        first), read out o = S^T q.  q, k, v [QH, D]; g, beta [QH]."""
        kS = np.einsum("hk,hkv->hv", k, S_prev)              # S_prev^T k
        S = np.exp(g)[:, None, None] * (S_prev - beta[:, None, None] * k[:, :, None] * kS[:, None, :]) \
            + beta[:, None, None] * k[:, :, None] * v[:, None, :]
        o = np.einsum("hkv,hk->hv", S, q)
        return o, S

    def recurrent_token(self, kind: int, qkv: np.ndarray, a: np.ndarray, S_prev: np.ndarray,
                        round_out: bool = True):
        """The token mixing of a recurrent layer from its projections (both
        already at their rounding point): ``qkv`` stacks q, k and v heads
        (QH*D values each), ``a`` the gate pre-activations and, for a delta
        layer, the write-strength pre-activations after them.  q and k are
        L2-normalised per head; the log-decay is log sigmoid(gate) and the
        write strength sigmoid(.).  Returns (read-out [QH*D] at its rounding
        point, or unrounded with ``round_out=False``; the new state held in
        fp32)."""
        s, r = self.s, self.r
        QH, D = s.n_qhead, s.head_dim
        q = r(self.l2norm(qkv[:QH * D].reshape(QH, D)))
        k = r(self.l2norm(qkv[QH * D:2 * QH * D].reshape(QH, D)))
        v = qkv[2 * QH * D:3 * QH * D].reshape(QH, D)
        if kind == RECUR:
            o, S = self.recur_mix(q, k, v, log_sigmoid(a[:QH]), S_prev)
        else:
            o, S = self.delta_mix(q, k, v, log_sigmoid(a[:QH]), sigmoid(a[QH:2 * QH]), S_prev)
        # the state is held in fp32 between tokens
        o = o.reshape(-1)
        return (r(o) if round_out else o), (S if self.exact else f32(S))

    def recurrent_layer(self, l: int, xn: np.ndarray, S_prev: np.ndarray):
        """Recurrent layer l on its normalised input row ``xn``: the stacked
        q/k/v projection (wqkv) and the gate projection (wa: gate rows, then a
        delta layer's write-strength rows), each rounded, then
        ``recurrent_token``."""
        p = f"layers.{l}."
        qkv = self.r(self.matvec(p + "wqkv", xn))
        a = self.r(self.matvec(p + "wa", xn))
        return self.recurrent_token(self.s.kinds[l], qkv, a, S_prev)

    def l2norm(self, x: np.ndarray) -> np.ndarray:
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + self.s.eps)

    def step(self, token: int, pos: int, prefix: Dict[int, Tuple[np.ndarray, np.ndarray]],
             states: Dict[int, np.ndarray]):
        """One token at position ``pos``.

        ``prefix[l]`` is (K, V) [KVH, L, D] of every earlier position of this
        path at attention layer l; ``states[l]`` is the recurrent state
        [QH, D, D] before this token at recurrent layer l.  Returns
        (logits [V], rows {l: (k, v)}, new_states {l: S}).
        """
        s = self.s
        r = self.r
        QH, KVH, D = s.n_qhead, s.n_kvhead, s.head_dim
        x = bf16_bits_to_f64(self.W["emb"][token])
        rows, new_states = {}, {}
        for l, kind in enumerate(s.kinds):
            p = f"layers.{l}."
            xn = r(self.rmsnorm(x, p + "attn_norm"))
            if kind == ATTN:
                qkv = r(self.matvec(p + "wqkv", xn))
                q = qkv[:QH * D].reshape(QH, D)
                k = qkv[QH * D:(QH + KVH) * D].reshape(KVH, D)
                v = qkv[(QH + KVH) * D:].reshape(KVH, D)
                q = r(self.rope(q, pos))
                k = r(self.rope(k, pos))
                Kp, Vp = prefix[l]
                Ka = np.concatenate([Kp, k[:, None, :]], axis=1)
                Va = np.concatenate([Vp, v[:, None, :]], axis=1)
                o = r(self.attention(q, Ka, Va).reshape(-1))
                rows[l] = (k, v)
            else:
                o, new_states[l] = self.recurrent_layer(l, xn, states[l])
            x = r(x + r(self.matvec(p + "wo", o)))
            hn = r(self.rmsnorm(x, p + "ffn_norm"))
            gt = r(self.matvec(p + "wg", hn))
            u = r(self.matvec(p + "wu", hn))
            act = r(gt / (1.0 + np.exp(-gt)) * u)     # silu(g) * u
            x = r(x + r(self.matvec(p + "wd", act)))
        xf = r(self.rmsnorm(x, "final_norm"))
        logits = self.matvec("head", xf)
        if not self.exact:
            logits = f32(logits)
        return logits, rows, new_states

    # -------------------------------------------------------- sequences

    def new_seq(self, cap: int, history: Optional[Sequence[int]] = None,
                kv: Optional[dict] = None, ctx_len: int = 0,
                s0: Optional[dict] = None) -> "Seq":
        return Seq(self, cap, history, kv, ctx_len, s0)

    def tree_scores(self, seq: "Seq", parents: Sequence[int], tokens: Sequence[int],
                    rows_wanted: Optional[Sequence[int]] = None) -> np.ndarray:
        """Brute-force scorer: logits [n, V] of every node, each the step of
        the node's token after the committed sequence and its ancestors.

        Nodes are visited in index order (parents come first); a node's KV
        rows and recurrent state are kept for its descendants.  With
        ``rows_wanted`` only those nodes and their ancestors are stepped
        (other rows are NaN).
        """
        n = len(parents)
        parents = [int(p) for p in parents]
        need = set(range(n)) if rows_wanted is None else set()
        if rows_wanted is not None:
            for i in rows_wanted:
                j = int(i)
                while j >= 0:
                    need.add(j)
                    j = parents[j]
        depth = [0] * n
        node_rows: List[Optional[dict]] = [None] * n
        node_state: List[Optional[dict]] = [None] * n
        out = np.full((n, self.s.vocab), np.nan)
        for i in range(n):
            if i > 0:
                if not (0 <= parents[i] < i):
                    raise ValueError("parents must precede children")
                depth[i] = depth[parents[i]] + 1
            if i not in need:
                continue
            anc = []
            j = parents[i]
            while j >= 0:
                anc.append(j)
                j = parents[j]
            anc.reverse()
            prefix = {}
            for l, kind in enumerate(self.s.kinds):
                if kind != ATTN:
                    continue
                K0, V0 = seq.K[l][:, :seq.ctx_len], seq.V[l][:, :seq.ctx_len]
                if anc:
                    Kt = np.stack([node_rows[a][l][0] for a in anc], axis=1)
                    Vt = np.stack([node_rows[a][l][1] for a in anc], axis=1)
                    K0 = np.concatenate([K0, Kt], axis=1)
                    V0 = np.concatenate([V0, Vt], axis=1)
                prefix[l] = (K0, V0)
            st = seq.S if parents[i] < 0 else node_state[parents[i]]
            logits, rows, new_st = self.step(int(tokens[i]), seq.ctx_len + depth[i], prefix, st)
            out[i] = logits
            node_rows[i] = rows
            node_state[i] = new_st
        return out


class Seq:
    """Committed state of one request: its KV rows, recurrent states and
    token history (prompt and every committed token)."""

    def __init__(self, model: Oracle, cap: int, history=None, kv=None, ctx_len=0, s0=None):
        s = model.s
        self.m = model
        self.cap = cap
        self.ctx_len = ctx_len
        self.history: List[int] = [] if history is None else [int(t) for t in history]
        self.K, self.V, self.S = {}, {}, {}
        for l, kind in enumerate(s.kinds):
            if kind == ATTN:
                K = np.zeros((s.n_kvhead, cap, s.head_dim))
                V = np.zeros((s.n_kvhead, cap, s.head_dim))
                if kv is not None and ctx_len > 0:
                    K[:, :ctx_len] = t2f64(kv[(l, "k")][:, :ctx_len])
                    V[:, :ctx_len] = t2f64(kv[(l, "v")][:, :ctx_len])
                self.K[l], self.V[l] = K, V
            else:
                if s0 is not None:
                    self.S[l] = t2f64(s0[l])
                else:
                    self.S[l] = np.zeros((s.n_qhead, s.head_dim, s.head_dim))

    def step(self, token: int) -> np.ndarray:
        """Append one token: its KV rows and states become committed."""
        if self.ctx_len >= self.cap:
            raise ValueError("sequence capacity exceeded")
        prefix = {l: (self.K[l][:, :self.ctx_len], self.V[l][:, :self.ctx_len]) for l in self.K}
        logits, rows, new_st = self.m.step(int(token), self.ctx_len, prefix, self.S)
        for l in self.K:
            self.K[l][:, self.ctx_len] = rows[l][0]
            self.V[l][:, self.ctx_len] = rows[l][1]
        self.S.update(new_st)
        self.ctx_len += 1
        self.history.append(int(token))
        return logits

    def commit(self, tokens: Sequence[int]) -> Optional[np.ndarray]:
        last = None
        for t in tokens:
            last = self.step(t)
        return last


# ------------------------------------------------------------ scores

def apply_modifiers(logits: np.ndarray, prior: Sequence[int], mods: Optional[Modifiers]) -> np.ndarray:
    """Modified fp32 scores of one row: repetition penalty over ``prior``
    (l/theta for l>0, else l*theta), then logit_bias, then the allow-mask
    (disallowed ids score -inf).  fp32 arithmetic, as the decision is taken
    on the fp32 logits."""
    s = np.asarray(logits, dtype=np.float64).astype(np.float32)
    if mods is None:
        return s
    th = np.float32(mods.rep_penalty)
    if mods.rep_penalty != 1.0 and len(prior):
        ids = np.unique(np.asarray(prior, dtype=np.int64))
        v = s[ids]
        s[ids] = np.where(v > 0, v / th, v * th).astype(np.float32)
    if len(mods.bias_ids):
        s[mods.bias_ids] = (s[mods.bias_ids] + mods.bias_vals.astype(np.float32)).astype(np.float32)
    if mods.allow_bits is not None:
        ids = np.arange(s.shape[0])
        allowed = (mods.allow_bits[ids // 32] >> (ids % 32).astype(np.uint32)) & 1
        s[allowed == 0] = np.float32(-np.inf)
    return s


def top2(scores: np.ndarray) -> Tuple[int, float, float, float]:
    """(argmax, top-1, top-2, gap in bf16 ulps of top-1).  The argmax is the
    lowest id among equal maxima; top-2 is the best score among the other
    ids (equal to top-1 on an exact tie)."""
    s = np.asarray(scores, dtype=np.float64)
    a = int(np.argmax(s))
    l1 = float(s[a])
    rest = np.concatenate([s[:a], s[a + 1:]])
    l2 = float(rest.max()) if rest.size else -np.inf
    if l2 == -np.inf:
        gap = np.inf
    else:
        gap = (l1 - l2) / float(ulp_bf16(l1))
    return a, l1, l2, gap


def path_tokens(parents: Sequence[int], tokens: Sequence[int], i: int) -> List[int]:
    out = []
    while i >= 0:
        out.append(int(tokens[i]))
        i = int(parents[i])
    return out[::-1]


def tree_decisions(logits: np.ndarray, parents, tokens, history: Sequence[int],
                   mods: Optional[Modifiers] = None):
    """Per-row (argmax, gap) on modified scores; a row's prior tokens are
    the history plus its path root..node."""
    n = len(parents)
    am = np.zeros(n, dtype=np.int32)
    gap = np.zeros(n)
    for i in range(n):
        prior = list(history) + path_tokens(parents, tokens, i)
        a, _, _, g = top2(apply_modifiers(logits[i], prior, mods))
        am[i], gap[i] = a, g
    return am, gap


def accept_walk(parents: Sequence[int], tokens: Sequence[int], argmax: Sequence[int]):
    """From the root, take the model's token and move to the child that
    carries it; stop where none does and keep the model's token there.
    Returns (path node indices, emitted tokens); len(emitted) == len(path)."""
    n = len(parents)
    kids: List[List[int]] = [[] for _ in range(n)]
    for i in range(1, n):
        kids[int(parents[i])].append(i)
    cur = 0
    path, emitted = [0], []
    while True:
        g = int(argmax[cur])
        emitted.append(g)
        nxt = [c for c in kids[cur] if int(tokens[c]) == g]
        if not nxt:
            break
        cur = nxt[0]
        path.append(cur)
    return path, emitted


def greedy(seq: Seq, first: int, k: int, mods: Optional[Modifiers] = None):
    """Plain greedy decoding: feed ``first``, then k-1 argmax tokens.
    Returns (tokens emitted [k], gaps [k]); ``seq`` ends having consumed
    ``first`` and the first k-1 emitted tokens."""
    out, gaps = [], []
    t = first
    for i in range(k):
        logits = seq.step(t)
        a, _, _, g = top2(apply_modifiers(logits, seq.history, mods))
        out.append(a)
        gaps.append(g)
        t = a
    return out, gaps


# ------------------------------------------------------------ sampling
#
# A sampled request (temperature T > 0) draws the token at sequence index t
# as the argmax of log p_t + G_t, where p_t is the distribution of the
# modified scores divided by T and G_t a vector of standard Gumbel noise
# from a generator keyed by (seed, t) ("Exactness", Sampling; "Drafters and
# tree verify", Sampling).  log p_t differs from scores/T by one constant
# per row, so the argmax is taken over fp32(fp32(scores / T) + G) directly.
#
# Sequence indices count from 0 at the first prompt token: a verify row
# whose node sits at position ctx_len + depth scores the token at index
# ctx_len + depth + 1, and plain decoding that has consumed c tokens draws
# index c.
#
# The generator is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
# random numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter, a
# 64-bit key, ten rounds.  Vocabulary id v takes word v % 4 of the block at
# counter (v // 4, t, 0, 0) under key (seed low word, seed high word); the
# word x becomes u = (x + 1/2) / 2^32, strictly inside (0, 1), and
# G = -log(-log u) is evaluated in fp64 and rounded to fp32.

_PH_M0, _PH_M1 = 0xD2511F53, 0xCD9E8D57    # round multipliers
_PH_W0, _PH_W1 = 0x9E3779B9, 0xBB67AE85    # key schedule increments
_U32 = 0xFFFFFFFF


class Sampling:
    """Temperature and 64-bit seed of one sampled request (T > 0)."""

    def __init__(self, temperature: float, seed: int):
        if not (temperature > 0 and math.isfinite(temperature)):
            raise ValueError("temperature must be positive and finite")
        self.temperature = float(temperature)
        self.seed = int(seed) & 0xFFFFFFFFFFFFFFFF


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> List[int]:
    """One Philox4x32-10 block, scalar: four 32-bit words of counter, two of
    key.  Each round multiplies words 0 and 2 by the two round constants,
    crosses the high halves of the products with words 1 and 3 and the key,
    and keeps the low halves; the key then advances by the Weyl increments."""
    c = [int(w) & _U32 for w in ctr]
    k0, k1 = int(key[0]) & _U32, int(key[1]) & _U32
    for _ in range(10):
        p0 = _PH_M0 * c[0]
        p1 = _PH_M1 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k0) & _U32, p1 & _U32,
             ((p0 >> 32) ^ c[3] ^ k1) & _U32, p0 & _U32]
        k0, k1 = (k0 + _PH_W0) & _U32, (k1 + _PH_W1) & _U32
    return c


def philox_words(seed: int, t: int, n: int) -> np.ndarray:
    """Words 0..n-1 of the stream (seed, t): word v is word v % 4 of the
    block at counter (v // 4, t, 0, 0).  The same rounds as philox4x32_10,
    one numpy lane per block."""
    nb = (n + 3) // 4
    c0 = np.arange(nb, dtype=np.uint64)
    c1 = np.full(nb, int(t) & _U32, dtype=np.uint64)
    c2 = np.zeros(nb, dtype=np.uint64)
    c3 = np.zeros(nb, dtype=np.uint64)
    k0, k1 = int(seed) & _U32, (int(seed) >> 32) & _U32
    m = np.uint64(_U32)
    for _ in range(10):
        p0 = np.uint64(_PH_M0) * c0
        p1 = np.uint64(_PH_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0)) & m, p1 & m, \
                         ((p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1)) & m, p0 & m
        k0, k1 = (k0 + _PH_W0) & _U32, (k1 + _PH_W1) & _U32
    return np.stack([c0, c1, c2, c3], axis=1).reshape(-1)[:n].astype(np.uint32)


def gumbel(seed: int, t: int, n: int) -> np.ndarray:
    """fp32 standard Gumbel noise G_t of the stream (seed, t), n values."""
    u = (philox_words(seed, t, n).astype(np.float64) + 0.5) * 2.0 ** -32
    return (-np.log(-np.log(u))).astype(np.float32)


def sample_keys(scores: np.ndarray, smp: Sampling, t: int) -> np.ndarray:
    """fp32 keys fp32(fp32(scores / T) + G_t) of one row; their argmax
    (lowest id on an exact tie) is the draw.  -inf scores stay -inf."""
    s = np.asarray(scores, dtype=np.float32)
    return (s / np.float32(smp.temperature) + gumbel(smp.seed, t, s.shape[0])).astype(np.float32)


def node_depths(parents: Sequence[int]) -> List[int]:
    d = [0] * len(parents)
    for i in range(1, len(parents)):
        d[i] = d[int(parents[i])] + 1
    return d


def sampled_tree_decisions(logits: np.ndarray, parents, tokens, history: Sequence[int], ctx_len: int,
                           smp: Sampling, mods: Optional[Modifiers] = None):
    """Per-row (draw, gap) of a sampled request: row i draws the token at
    index ctx_len + depth(i) + 1 from its modified scores.  The gap is the
    top-1/top-2 key difference in bf16 ulps of the top key."""
    n = len(parents)
    dep = node_depths(parents)
    am = np.zeros(n, dtype=np.int32)
    gap = np.zeros(n)
    for i in range(n):
        prior = list(history) + path_tokens(parents, tokens, i)
        keys = sample_keys(apply_modifiers(logits[i], prior, mods), smp, ctx_len + dep[i] + 1)
        a, _, _, g = top2(keys)
        am[i], gap[i] = a, g
    return am, gap


def sampled(seq: Seq, first: int, k: int, smp: Sampling, mods: Optional[Modifiers] = None):
    """Plain sampled decoding: feed ``first``, then k-1 drawn tokens; the
    draw after c consumed tokens is index c.  Returns (tokens [k], gaps)."""
    out, gaps = [], []
    t = first
    for _ in range(k):
        logits = seq.step(t)
        keys = sample_keys(apply_modifiers(logits, seq.history, mods), smp, seq.ctx_len)
        a, _, _, g = top2(keys)
        out.append(a)
        gaps.append(g)
        t = a
    return out, gaps


# ------------------------------------------------- residual tree sampling
#
# Deterministic-candidate residual sampling ("Algorithm and correctness
# contract", Deterministic tree candidates and residual verification): at a
# node with target distribution p (softmax of the modified scores over T),
# the children are tried in index order; a candidate x is accepted with
# probability r(x), r starting at p; a rejected candidate's mass is removed
# and r renormalised; when every candidate fails, the replacement is drawn
# from the residual r and the round ends.
#
# Reading taken here: a visited node consumes ONE uniform u, the uniform of
# its depth.  Trying the candidates in order with u rescaled after each
# rejection, then drawing the residual with the rescaled u by inverse CDF in
# token-id order, is exactly inverse-CDF sampling of p over the order
# (candidates in index order, then every other id ascending): the first
# position where the running sum of the weights exceeds u times their total.
# A leaf (no candidates) draws from p, which gives the next round its root.

def residual_weights(scores: np.ndarray, temperature: float) -> np.ndarray:
    """Unnormalised fp64 weights exp(s/T - max) of fp32 scores (-inf -> 0)."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64) / float(temperature)
    fin = np.isfinite(s)
    w = np.zeros_like(s)
    w[fin] = np.exp(s[fin] - s[fin].max())
    return w


def residual_decision(scores: np.ndarray, candidates: Sequence[int], temperature: float, u: float):
    """('accept', j) for candidate j, or ('emit', token), with the margin
    |running sum - u * total| / total at the decision (for tie checks)."""
    w = residual_weights(scores, temperature)
    cand = [int(c) for c in candidates]
    rest = np.ones(w.shape[0], dtype=bool)
    rest[cand] = False
    order = np.concatenate([np.asarray(cand, dtype=np.int64), np.nonzero(rest)[0]])
    cum = np.cumsum(w[order])
    total = math.fsum(w)
    thr = u * total
    pos = int(np.searchsorted(cum, thr, side="right"))
    pos = min(pos, order.shape[0] - 1)
    while w[order[pos]] == 0.0 and pos > 0:     # never land on a zero-weight id
        pos -= 1
    lo = cum[pos - 1] if pos > 0 else 0.0
    margin = min(abs(cum[pos] - thr), abs(thr - lo)) / total
    if pos < len(cand):
        return ("accept", pos), margin
    return ("emit", int(order[pos])), margin


def residual_walk(logits: np.ndarray, parents, tokens, history: Sequence[int], temperature: float,
                  uniforms: Sequence[float], mods: Optional[Modifiers] = None):
    """One round of residual tree sampling: (path node ids, emitted tokens,
    the smallest decision margin).  uniforms[d] is the uniform of depth d."""
    n = len(parents)
    kids: List[List[int]] = [[] for _ in range(n)]
    for i in range(1, n):
        kids[int(parents[i])].append(i)
    cur, d = 0, 0
    path, emitted, margin = [0], [], 1.0
    while True:
        prior = list(history) + path_tokens(parents, tokens, cur)
        scores = apply_modifiers(logits[cur], prior, mods)
        (kind, val), mg = residual_decision(scores, [int(tokens[c]) for c in kids[cur]], temperature,
                                            float(uniforms[d]))
        margin = min(margin, mg)
        if kind == "emit":
            emitted.append(val)
            return path, emitted, margin
        cur = kids[cur][val]
        path.append(cur)
        emitted.append(int(tokens[cur]))
        d += 1
