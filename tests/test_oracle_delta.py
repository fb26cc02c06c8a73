"""Pins of the oracle's gated delta rule (the pages' Gated DeltaNet layers).

The oracle steps S = alpha (I - beta k k^T) S_parent + beta k v^T one token at
a time (``Oracle.delta_mix``).  These tests hold that loop to what the
mathematics and the pages fix:

* the defining property of the delta rule: for a unit key k the state's
  answer to k moves a fraction beta of the way to v (after the decay alpha),
  and its answer to any key orthogonal to k only decays;
* the pseudo-value form ("Drafters and tree verify", Tree verify through
  recurrent layers): with u_t the solution of a unit lower-triangular system
  whose off-diagonal part is ancestor-masked,
      (I + A) u = beta * (v - e^{gc} S0^T k),
      A[t, s] = beta_t e^{gc_t - gc_s} (k_t . k_s)   for s a strict ancestor of t,
  the state after any root-to-node path is
      S_path = e^{gc_last} S0 + sum_{t in path} e^{gc_last - gc_t} k_t (x) u_t
  and the read-out is o_t = e^{gc_t} S0^T q_t + sum_{s in anc*(t)} e^{gc_t - gc_s} (q_t . k_s) u_s;
* the inverse of the ancestor-masked matrix is ancestor-masked too, so u_t
  depends only on t's own path;
* tree rows of a small hybrid model with delta layers equal the sequential
  decode of each node's path.
"""
import numpy as np

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
    beta = oracle.sigmoid(rng.standard_normal((T, QH)) * 2.0)
    S0 = rng.standard_normal((QH, D, D))
    return q, k, v, g, beta, S0


def test_sigmoid():
    a = np.linspace(-40, 40, 161)
    np.testing.assert_allclose(oracle.sigmoid(a), 1.0 / (1.0 + np.exp(-a)), rtol=1e-14)


def test_delta_rule_moves_the_answer_to_k_toward_v():
    q, k, v, g, beta, S0 = _inputs(1, 0)
    _, S = oracle.Oracle.delta_mix(q[0], k[0], v[0], g[0], beta[0], S0)
    rng = np.random.default_rng(1)
    for h in range(QH):
        a, b, kk = np.exp(g[0, h]), beta[0, h], k[0, h]
        old = S0[h].T @ kk
        np.testing.assert_allclose(S[h].T @ kk, a * ((1 - b) * old) + b * v[0, h], rtol=1e-12, atol=1e-12)
        x = rng.standard_normal(D)
        x -= (x @ kk) * kk                                  # orthogonal to k
        np.testing.assert_allclose(S[h].T @ x, a * (S0[h].T @ x), rtol=1e-12, atol=1e-12)
    # beta = 1, no decay: the state returns v for k exactly
    _, S1 = oracle.Oracle.delta_mix(q[0], k[0], v[0], np.zeros(QH), np.ones(QH), S0)
    for h in range(QH):
        np.testing.assert_allclose(S1[h].T @ k[0, h], v[0, h], rtol=1e-12, atol=1e-12)
    # beta = 0: decay only
    _, S2 = oracle.Oracle.delta_mix(q[0], k[0], v[0], g[0], np.zeros(QH), S0)
    np.testing.assert_allclose(S2, np.exp(g[0])[:, None, None] * S0, rtol=1e-14)


def _pseudo_values(parents, k, v, g, beta, S0, h):
    """u of every node for head h from the ancestor-masked system, by a
    library solve of the whole matrix; also returns gc and the inverse."""
    n = len(parents)
    anc = np.zeros((n, n), dtype=bool)        # anc[t, s]: s is an ancestor of t or t itself
    gc = np.zeros(n)
    for t in range(n):
        p = parents[t]
        if p >= 0:
            anc[t] = anc[p]
            gc[t] = gc[p]
        anc[t, t] = True
        gc[t] += g[t, h]
    strict = anc & ~np.eye(n, dtype=bool)
    A = np.where(strict, beta[:, h, None] * np.exp(gc[:, None] - gc[None, :]) * (k[:, h] @ k[:, h].T), 0.0)
    rhs = beta[:, h, None] * (v[:, h] - np.exp(gc)[:, None] * (k[:, h] @ S0[h]))
    M = np.eye(n) + A
    u = np.linalg.solve(M, rhs)
    return u, gc, anc, np.linalg.inv(M)


def _closed_state(path, k, u, gc, S0h, h):
    want = np.exp(gc[path[-1]]) * S0h
    for t in path:
        want = want + np.exp(gc[path[-1]] - gc[t]) * np.outer(k[t, h], u[t])
    return want


def test_chain_loop_matches_pseudo_value_form():
    T = 9
    q, k, v, g, beta, S0 = _inputs(T, 2)
    parents = list(range(-1, T - 1))
    S, outs = S0, []
    for t in range(T):
        o, S = oracle.Oracle.delta_mix(q[t], k[t], v[t], g[t], beta[t], S)
        outs.append(o)
    for h in range(QH):
        u, gc, _, _ = _pseudo_values(parents, k, v, g, beta, S0, h)
        for t in range(T):
            want = np.exp(gc[t]) * (S0[h].T @ q[t, h])
            for s in range(t + 1):
                want = want + np.exp(gc[t] - gc[s]) * (q[t, h] @ k[s, h]) * u[s]
            np.testing.assert_allclose(outs[t][h], want, rtol=1e-10, atol=1e-10)
        np.testing.assert_allclose(S[h], _closed_state(list(range(T)), k, u, gc, S0[h], h),
                                   rtol=1e-10, atol=1e-10)


def test_closed_form_and_masked_inverse_for_every_tree_path():
    parents = synth.random_tree(14, 5)
    n = len(parents)
    q, k, v, g, beta, S0 = _inputs(n, 3)
    states, outs = [], []
    for i in range(n):
        Sp = S0 if parents[i] < 0 else states[parents[i]]
        o, S = oracle.Oracle.delta_mix(q[i], k[i], v[i], g[i], beta[i], Sp)
        states.append(S)
        outs.append(o)
    for h in range(QH):
        u, gc, anc, inv = _pseudo_values(parents, k, v, g, beta, S0, h)
        # the inverse keeps the ancestor mask: u_t depends on t's path only
        assert np.all(inv[~anc] == 0.0) or np.abs(inv[~anc]).max() < 1e-14
        for i in range(n):
            path = [j for j in range(n) if anc[i, j]]          # root..i in index order
            np.testing.assert_allclose(states[i][h], _closed_state(path, k, u, gc, S0[h], h),
                                       rtol=1e-10, atol=1e-10)
            want = np.exp(gc[i]) * (S0[h].T @ q[i, h])
            for s in path:
                want = want + np.exp(gc[i] - gc[s]) * (q[i, h] @ k[s, h]) * u[s]
            np.testing.assert_allclose(outs[i][h], want, rtol=1e-10, atol=1e-10)


HYBD = synth.scaled(synth.C0, "c0_delta", n_layer=4, kinds=[2, 2, 2, 0])


def test_delta_hybrid_tree_rows_equal_sequential_decode():
    w = synth.weights(HYBD, seed=1)
    assert w["layers.0.wa"].shape == (2 * HYBD.n_qhead, HYBD.hidden)
    orc = oracle.Oracle(HYBD, w)
    s0 = synth.state0(HYBD, seed=6)
    assert sorted(s0) == [0, 1, 2]
    prompt = synth.uniform_ids(6, HYBD.vocab, 3)
    base = orc.new_seq(cap=64, s0=s0)
    base.commit(prompt)
    parents = synth.spine_tree(10, 1)
    tokens = synth.tree_tokens(parents, HYBD.vocab, 2, root_token=9)
    rows = orc.tree_scores(base, parents, tokens)
    for i in range(len(parents)):
        s = orc.new_seq(cap=64, s0=s0)
        s.commit(prompt)
        last = s.commit(oracle.path_tokens(parents, tokens, i))
        np.testing.assert_array_equal(rows[i], last)
    # the delta layers change the model: the same weights read as a plain
    # gated recurrence (gate rows only) give other logits
    plain = synth.scaled(synth.C0, "c0_hybrid_plain", n_layer=4, kinds=[1, 1, 1, 0])
    w2 = dict(w)
    for l in range(3):
        w2[f"layers.{l}.wa"] = w[f"layers.{l}.wa"][:HYBD.n_qhead]
    plain_logits = oracle.Oracle(plain, w2).new_seq(cap=64, s0=s0).commit(prompt)
    delta_logits = orc.new_seq(cap=64, s0=s0).commit(prompt)
    assert not np.allclose(plain_logits, delta_logits)


def test_delta_state_is_fp32_and_finite():
    w = synth.weights(HYBD, seed=1)
    orc = oracle.Oracle(HYBD, w)
    seq = orc.new_seq(cap=64, s0=synth.state0(HYBD, seed=6))
    seq.commit(synth.uniform_ids(20, HYBD.vocab, 3))
    for l, S in seq.S.items():
        assert np.isfinite(S).all()
        np.testing.assert_array_equal(oracle.f32(S), S)
