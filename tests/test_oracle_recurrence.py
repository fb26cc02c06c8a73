"""Pins of the oracle's gated linear recurrence.

The oracle advances the state one token at a time (S = e^g S_parent + k v^T,
o = S^T q).  These tests hold that loop to two other forms fixed by the
mathematics and the pages:

* the parallel (attention-like) form of a gated linear recurrence,
  o_t = e^{gc_t} S0^T q_t + sum_{s<=t} e^{gc_t - gc_s} (q_t . k_s) v_s,
  with gc the cumulative log-gate along the path;
* the closed form of the state after a path ("Drafters and tree verify",
  Tree verify through recurrent layers):
  S_path = e^{gc_last} S0 + sum_{t in path} e^{gc_last - gc_t} k_t (x) v_t,
  which holds for every root-to-node path of a tree.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

QH, D = 3, 8


def _inputs(T, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, QH, D))
    k = rng.standard_normal((T, QH, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, QH, D))
    g = oracle.log_sigmoid(rng.standard_normal((T, QH)) * 1.5)
    S0 = rng.standard_normal((QH, D, D))
    return q, k, v, g, S0


def test_chain_loop_matches_parallel_form():
    T = 9
    q, k, v, g, S0 = _inputs(T, 0)
    S = S0
    outs = []
    for t in range(T):
        o, S = oracle.Oracle.recur_mix(q[t], k[t], v[t], g[t], S)
        outs.append(o)
    gc = np.cumsum(g, axis=0)                              # [T, QH]
    for t in range(T):
        for h in range(QH):
            want = np.exp(gc[t, h]) * (S0[h].T @ q[t, h])
            for s in range(t + 1):
                want = want + np.exp(gc[t, h] - gc[s, h]) * (q[t, h] @ k[s, h]) * v[s, h]
            np.testing.assert_allclose(outs[t][h], want, rtol=1e-12, atol=1e-12)
    # closed form of the final state
    for h in range(QH):
        want = np.exp(gc[-1, h]) * S0[h]
        for t in range(T):
            want = want + np.exp(gc[-1, h] - gc[t, h]) * np.outer(k[t, h], v[t, h])
        np.testing.assert_allclose(S[h], want, rtol=1e-12, atol=1e-12)


def test_closed_form_holds_for_every_tree_path():
    parents = synth.random_tree(12, 4)
    n = len(parents)
    q, k, v, g, S0 = _inputs(n, 1)
    states = []
    for i in range(n):
        Sp = S0 if parents[i] < 0 else states[parents[i]]
        _, S = oracle.Oracle.recur_mix(q[i], k[i], v[i], g[i], Sp)
        states.append(S)
    for i in range(n):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parents[j]
        path.reverse()
        gc = np.cumsum(g[path], axis=0)
        for h in range(QH):
            want = np.exp(gc[-1, h]) * S0[h]
            for d, t in enumerate(path):
                want = want + np.exp(gc[-1, h] - gc[d, h]) * np.outer(k[t, h], v[t, h])
            np.testing.assert_allclose(states[i][h], want, rtol=1e-12, atol=1e-12)


def test_single_step_special_case():
    # n = 1 from a zero state: o = (q . k) v
    q, k, v, g, _ = _inputs(1, 2)
    o, S = oracle.Oracle.recur_mix(q[0], k[0], v[0], g[0], np.zeros((QH, D, D)))
    for h in range(QH):
        np.testing.assert_allclose(o[h], (q[0, h] @ k[0, h]) * v[0, h], rtol=1e-13)


def test_log_sigmoid_and_l2norm():
    a = np.linspace(-30, 30, 301)
    want = torch.nn.functional.logsigmoid(torch.from_numpy(a)).numpy()
    np.testing.assert_allclose(oracle.log_sigmoid(a), want, rtol=1e-14, atol=1e-300)
    m = oracle.Oracle.__new__(oracle.Oracle)
    m.s = synth.C0
    x = np.random.default_rng(0).standard_normal((5, 64)) * 3
    y = m.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(y / np.linalg.norm(y, axis=-1, keepdims=True),
                               x / np.linalg.norm(x, axis=-1, keepdims=True), rtol=1e-12)


HYB = synth.scaled(synth.C0, "c0_hybrid", n_layer=4, kinds=[1, 1, 1, 0])


def test_hybrid_tree_rows_equal_sequential_decode():
    w = synth.weights(HYB, seed=1)
    orc = oracle.Oracle(HYB, w)
    s0 = synth.state0(HYB, seed=6)
    prompt = synth.uniform_ids(6, HYB.vocab, 3)
    base = orc.new_seq(cap=64, s0=s0)
    base.commit(prompt)
    parents = synth.spine_tree(10, 1)
    tokens = synth.tree_tokens(parents, HYB.vocab, 2, root_token=9)
    rows = orc.tree_scores(base, parents, tokens)
    for i in range(len(parents)):
        s = orc.new_seq(cap=64, s0=s0)
        s.commit(prompt)
        last = s.commit(oracle.path_tokens(parents, tokens, i))
        np.testing.assert_array_equal(rows[i], last)


def test_hybrid_state_is_fp32_and_finite():
    w = synth.weights(HYB, seed=1)
    orc = oracle.Oracle(HYB, w)
    seq = orc.new_seq(cap=64, s0=synth.state0(HYB, seed=6))
    seq.commit(synth.uniform_ids(20, HYB.vocab, 3))
    for l, S in seq.S.items():
        assert np.isfinite(S).all()
        np.testing.assert_array_equal(oracle.f32(S), S)
