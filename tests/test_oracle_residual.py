"""Pins of the oracle's residual tree sampler ("Algorithm and correctness
contract", Deterministic tree candidates and residual verification; Evidence).

* The pages' exact enumeration counts (tests/golden/residual_enumeration.txt):
  a single-path candidate of probability 0.25 is accepted 2500 times of 10000
  on a Cartesian grid of two draws; a two-level tree's first two tokens come
  out [2000, 500, 3000, 4500] times.
* The oracle's one-uniform inverse-CDF form equals the procedure as the page
  states it (accept x with probability r(x), on rejection remove x and
  renormalise, after the last candidate draw the residual), run step by
  step with the uniform rescaled after each rejection.
* A replacement is never a candidate; over many draws the first two tokens
  of residual rounds follow the model's own p(x0) p(x1 | x0).
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "residual_enumeration.txt")
GRID = [(i + 0.5) / 100 for i in range(100)]


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            out[k] = [int(x) for x in v]
    return out


def _logits(p):
    return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


def test_enumeration_counts():
    g = _golden()
    # single path: root row p = [0.25, 0.75], one candidate (token 0)
    parents, tokens = [-1, 0], [1, 0]
    rows = np.stack([_logits([0.25, 0.75]), _logits([0.8, 0.2])])
    acc = 0
    for u1, u2 in itertools.product(GRID, GRID):
        path, _, _ = oracle.residual_walk(rows, parents, tokens, [], 1.0, [u1, u2])
        acc += len(path) > 1
    assert [acc, 100 * 100] == g["single_path"]
    # two levels: both tokens are candidates under the root, each a leaf
    parents, tokens = [-1, 0, 0], [1, 0, 1]
    rows = np.stack([_logits([0.25, 0.75]), _logits([0.8, 0.2]), _logits([0.4, 0.6])])
    counts = np.zeros(4, dtype=np.int64)
    for u1, u2 in itertools.product(GRID, GRID):
        _, emitted, _ = oracle.residual_walk(rows, parents, tokens, [], 1.0, [u1, u2])
        counts[2 * emitted[0] + emitted[1]] += 1
    assert counts.tolist() == g["two_level"]


def _stepwise(scores, candidates, T, u):
    """The page's procedure, literally: r starts as p; candidate x accepted
    with probability r(x) (u < r(x)), else x removed, r renormalised and u
    rescaled to the rejection event; after the last candidate the residual
    is drawn by inverse CDF in token-id order."""
    w = oracle.residual_weights(scores, T)
    r = w / math.fsum(w)
    for j, x in enumerate(candidates):
        if u < r[x]:
            return ("accept", j)
        u = (u - r[x]) / (1.0 - r[x])
        r = r.copy()
        r[x] = 0.0
        r = r / math.fsum(r)
    c = 0.0
    for v in range(r.shape[0]):
        c += r[v]
        if c > u and r[v] > 0:
            return ("emit", v)
    return ("emit", int(np.nonzero(r)[0][-1]))


def test_one_uniform_form_equals_the_stepwise_procedure():
    rng = np.random.default_rng(0)
    checked = 0
    for case in range(400):
        V = int(rng.integers(2, 40))
        s = (rng.normal(0, 2.0, V)).astype(np.float32)
        if case % 5 == 0:
            s[rng.integers(0, V)] = -np.inf
        k = int(rng.integers(0, min(V, 6)))
        cands = [int(c) for c in rng.choice(V, size=k, replace=False)]
        T = float(rng.choice([0.5, 1.0, 1.7]))
        u = float(rng.random())
        got, margin = oracle.residual_decision(s, cands, T, u)
        if margin < 1e-9:
            continue
        assert got == _stepwise(s, cands, T, u), (case, got)
        if got[0] == "emit":
            assert got[1] not in cands
        checked += 1
    assert checked > 350


def test_two_token_law_of_residual_rounds():
    """First two tokens of residual rounds (random candidate trees, random
    uniforms) against p(x0) p(x1 | x0) of a small model."""
    sh = synth.scaled(synth.C0, "c0_v16r", n_layer=1, vocab=16)
    orc = oracle.Oracle(sh, synth.weights(sh, seed=4))
    T = 1.1
    prompt = [2, 7, 1, 8, 2, 8]
    base = orc.new_seq(cap=32)
    base.commit(prompt[:-1])

    def clone(seq):
        s = orc.new_seq(cap=seq.cap)
        s.ctx_len, s.history = seq.ctx_len, list(seq.history)
        s.K = {l: v.copy() for l, v in seq.K.items()}
        s.V = {l: v.copy() for l, v in seq.V.items()}
        s.S = {l: v.copy() for l, v in seq.S.items()}
        return s

    def softmax(l):
        z = np.asarray(l, np.float32).astype(np.float64) / T
        z = np.exp(z - z.max())
        return z / z.sum()

    s0 = clone(base)
    p0 = softmax(s0.step(prompt[-1]))
    p1 = np.zeros((16, 16))
    for a in range(16):
        s = clone(base)
        s.step(prompt[-1])
        p1[a] = softmax(s.step(a))
    joint = (p0[:, None] * p1).reshape(-1)
    rng = np.random.default_rng(9)
    counts = np.zeros(256, dtype=np.int64)
    n_rounds = 2500
    parents = [-1, 0, 0, 1]
    for r in range(n_rounds):
        tokens = synth.tree_tokens(np.asarray(parents), 16, 1000 + r, prompt[-1])
        seq = clone(base)
        out = []
        root = prompt[-1]
        while len(out) < 2:
            tk = tokens.copy()
            tk[0] = root
            logits = orc.tree_scores(seq, parents, tk)
            path, emitted, _ = oracle.residual_walk(logits, parents, tk, seq.history, T, rng.random(4))
            seq.commit([int(tk[i]) for i in path])
            out += emitted
            root = emitted[-1]
        counts[out[0] * 16 + out[1]] += 1
    exp = n_rounds * joint
    big = exp >= 5
    p = stats.chisquare(np.append(counts[big], counts[~big].sum()),
                        np.append(exp[big], exp[~big].sum())).pvalue
    assert p > 1e-3, p
