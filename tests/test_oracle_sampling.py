"""Pins of the oracle's sampled verify.

"Exactness", Sampling and "Drafters and tree verify", Sampling: a sampled
request draws the target's own token at every verified node; a drafted token
survives while the draw lands on it.  With a seed, the token at sequence
index t is the argmax of log p_t + G_t, G_t Gumbel noise from a generator
keyed by (seed, t), an exact draw from p_t; the text of a seed is therefore
the same whatever the drafter proposed.

The pins: the generator's published known-answer vectors; the Gumbel law of
the noise (Kolmogorov-Smirnov, mean, variance); the Gumbel-max draw against
softmax(scores / T) by chi-square (planted mistakes -- the noise's sign, the
temperature's direction -- fail the same test); the greedy limit at small T;
and whole sampled rounds on the tiny model against plain sampled decoding,
for right, wrong and random drafters, with and without score modifiers, plus
the joint law of two emitted tokens against the model's own probabilities.
"""
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        ctr, key, out = (list(int(w, 16) for w in part.split()) for part in line.split("|"))
        rows.append((ctr, key, out))
    return rows


def test_philox_known_answers():
    rows = _kat()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert oracle.philox4x32_10(ctr, key) == out


def test_philox_stream_layout_matches_blocks():
    seed = 0x0123456789ABCDEF
    for t in (0, 1, 4097, 0xFFFFFFFF):
        w = oracle.philox_words(seed, t, 4 * 9 + 3)
        for v in range(w.shape[0]):
            blk = oracle.philox4x32_10([v // 4, t, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
            assert int(w[v]) == blk[v % 4]


def test_uniform_endpoints_are_open():
    # x = 0 and x = 2^32 - 1 map strictly inside (0, 1); G stays finite
    for x in (0, 2 ** 32 - 1):
        u = (x + 0.5) * 2.0 ** -32
        assert 0.0 < u < 1.0
        g = -math.log(-math.log(u))
        assert math.isfinite(g)
    assert -math.log(-math.log(0.5 * 2.0 ** -32)) > -3.2
    assert -math.log(-math.log(1 - 0.5 * 2.0 ** -32)) < 23.0


def test_gumbel_law():
    g = np.concatenate([oracle.gumbel(7, t, 50000).astype(np.float64) for t in range(4)])
    ks = stats.kstest(g, lambda x: np.exp(-np.exp(-x)))
    assert ks.pvalue > 1e-3, ks
    assert abs(g.mean() - np.euler_gamma) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.03
    # distinct (seed, t) give distinct streams
    assert not np.array_equal(oracle.gumbel(7, 0, 64), oracle.gumbel(7, 1, 64))
    assert not np.array_equal(oracle.gumbel(7, 0, 64), oracle.gumbel(8, 0, 64))
    assert not np.array_equal(oracle.gumbel(7, 0, 64), oracle.gumbel(7 + (1 << 32), 0, 64))


SCORES = np.array([1.25, -0.5, 2.0, 0.0, -np.inf, 1.9, -3.0], dtype=np.float32)


def _draw_counts(keyfn, n_draws, seed=11):
    counts = np.zeros(SCORES.shape[0], dtype=np.int64)
    for t in range(n_draws):
        counts[int(np.argmax(keyfn(t)))] += 1
    return counts


def _chi2_p(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0
    return stats.chisquare(counts[keep], counts.sum() * probs[keep]).pvalue


def _softmax(s, T):
    z = s.astype(np.float64) / T
    z = np.exp(z - z[np.isfinite(z)].max())
    return z / z.sum()


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_gumbel_max_draws_follow_softmax(T):
    smp = oracle.Sampling(T, 11)
    n = 20000
    counts = _draw_counts(lambda t: oracle.sample_keys(SCORES, smp, t), n)
    assert counts[4] == 0                       # a masked id is never drawn
    assert _chi2_p(counts, _softmax(SCORES, T)) > 1e-3


def test_planted_mistakes_fail_the_law():
    T, n = 1.0, 20000
    probs = _softmax(SCORES, T)

    def flipped(t):    # noise subtracted instead of added
        return SCORES / np.float32(T) - oracle.gumbel(11, t, SCORES.shape[0])

    def times_t(t):    # scores multiplied by T = 0.5 instead of divided
        return SCORES * np.float32(0.5) + oracle.gumbel(11, t, SCORES.shape[0])

    assert _chi2_p(_draw_counts(flipped, n), probs) < 1e-6
    assert _chi2_p(_draw_counts(times_t, n), _softmax(SCORES, 0.5)) < 1e-6


def test_small_temperature_is_greedy():
    rng = np.random.default_rng(5)
    for t in range(200):
        s = rng.normal(0, 3, 512).astype(np.float32)
        top = np.sort(s)[-2:]
        if top[1] - top[0] < 0.05:
            continue
        keys = oracle.sample_keys(s, oracle.Sampling(1e-3, 99), t)
        assert int(np.argmax(keys)) == int(np.argmax(s))


def test_sampling_rejects_bad_temperature():
    for T in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle.Sampling(T, 1)


# ---------------------------------------------------------- whole rounds

@pytest.fixture(scope="module")
def c0():
    return oracle.Oracle(synth.C0, synth.weights(synth.C0, seed=0))


def _plain(orc, prompt, first, k, smp, mods=None):
    s = orc.new_seq(cap=256)
    s.commit(prompt)
    return oracle.sampled(s, first, k, smp, mods)[0]


def _rounds(orc, prompt, first, n_tokens, drafter, parents, smp, mods=None, seq=None):
    if seq is None:
        seq = orc.new_seq(cap=256)
        seq.commit(prompt)
    root, out, per_round, r = first, [], [], 0
    while len(out) < n_tokens:
        tokens = drafter(seq, root, parents, r)
        logits = orc.tree_scores(seq, parents, tokens)
        am, _ = oracle.sampled_tree_decisions(logits, parents, tokens, seq.history, seq.ctx_len, smp, mods)
        path, emitted = oracle.accept_walk(parents, tokens, am)
        seq.commit([int(tokens[i]) for i in path])
        out += emitted
        per_round.append(len(emitted))
        root, r = emitted[-1], r + 1
    return out[:n_tokens], per_round


def _copy(orc, seq):
    s = orc.new_seq(cap=seq.cap)
    s.commit(seq.history)
    return s


def _clone(orc, seq):
    """The same committed state without stepping it again."""
    s = orc.new_seq(cap=seq.cap)
    s.ctx_len, s.history = seq.ctx_len, list(seq.history)
    s.K = {l: v.copy() for l, v in seq.K.items()}
    s.V = {l: v.copy() for l, v in seq.V.items()}
    s.S = {l: v.copy() for l, v in seq.S.items()}
    return s


def _right_drafter(orc, smp, mods, keep=0.7, seed=7):
    """Drafts the request's own sampled continuation along the spine, kept
    with probability ``keep`` a depth; other nodes random."""
    rng = np.random.default_rng(seed)

    def drafter(seq, root, parents, r):
        spine = synth.spine_nodes(parents)
        cont = oracle.sampled(_copy(orc, seq), root, len(spine) - 1, smp, mods)[0]
        forced = {}
        for d, node in enumerate(spine[1:]):
            if rng.random() >= keep:
                break
            forced[node] = cont[d]
        return synth.tree_tokens(parents, orc.s.vocab, 300 + r, root, forced)
    return drafter


def _wrong_drafter(orc, smp, mods):
    """Every drafted token differs from the draw at its parent."""
    def drafter(seq, root, parents, r):
        s = _copy(orc, seq)
        toks = synth.tree_tokens(parents, orc.s.vocab, 400 + r, root)
        dep = oracle.node_depths(parents)
        for i in range(1, len(parents)):
            p = int(parents[i])
            logits = orc.tree_scores(s, parents, toks, rows_wanted=[p])
            prior = s.history + oracle.path_tokens(parents, toks, p)
            keys = oracle.sample_keys(oracle.apply_modifiers(logits[p], prior, mods), smp,
                                      s.ctx_len + dep[p] + 1)
            draw = oracle.top2(keys)[0]
            sib = {int(toks[j]) for j in range(1, i) if parents[j] == p}
            t = int(toks[i])
            while t == draw or t in sib:
                t = (t + 1) % orc.s.vocab
            toks[i] = t
        return toks
    return drafter


def _random_drafter(orc):
    def drafter(seq, root, parents, r):
        return synth.tree_tokens(parents, orc.s.vocab, 500 + r, root)
    return drafter


@pytest.mark.parametrize("kind", ["right", "wrong", "random"])
def test_sampled_rounds_write_plain_sampled_text(c0, kind):
    smp = oracle.Sampling(0.8, 0xC0FFEE12345)
    prompt = synth.uniform_ids(48, synth.C0.vocab, 3)
    parents = synth.c0_tree()
    drafter = {"right": _right_drafter(c0, smp, None), "wrong": _wrong_drafter(c0, smp, None),
               "random": _random_drafter(c0)}[kind]
    got, per_round = _rounds(c0, prompt[:-1], int(prompt[-1]), 14, drafter, parents, smp)
    want = _plain(c0, prompt[:-1], int(prompt[-1]), 14, smp)
    assert got == want
    if kind == "right":
        assert max(per_round) > 1
    if kind == "wrong":
        assert per_round == [1] * len(per_round)


def test_sampled_text_depends_on_seed_not_on_greedy(c0):
    prompt = synth.uniform_ids(48, synth.C0.vocab, 3)
    a = _plain(c0, prompt[:-1], int(prompt[-1]), 12, oracle.Sampling(1.0, 1))
    b = _plain(c0, prompt[:-1], int(prompt[-1]), 12, oracle.Sampling(1.0, 2))
    s = c0.new_seq(cap=256)
    s.commit(prompt[:-1])
    g = oracle.greedy(s, int(prompt[-1]), 12)[0]
    assert a != b and a != g


def test_sampled_rounds_with_modifiers(c0):
    smp = oracle.Sampling(1.3, 77)
    mods = synth.modifiers(synth.C0.vocab, seed=4, n_bias=32, penalty=1.3, allow_frac=0.4)
    prompt = synth.uniform_ids(40, synth.C0.vocab, 5)
    parents = synth.c0_tree()
    got, _ = _rounds(c0, prompt[:-1], int(prompt[-1]), 10, _right_drafter(c0, smp, mods, seed=9),
                     parents, smp, mods)
    want = _plain(c0, prompt[:-1], int(prompt[-1]), 10, smp, mods)
    assert got == want
    ids = np.asarray(got)
    assert np.all((mods.allow_bits[ids // 32] >> (ids % 32).astype(np.uint32)) & 1)


def test_two_token_law_of_sampled_rounds():
    """Over many seeds, the first two tokens of sampled tree rounds (random
    drafter, small vocabulary) follow p(x0) p(x1 | x0) of the model itself."""
    sh = synth.scaled(synth.C0, "c0_v16", n_layer=1, vocab=16)
    orc = oracle.Oracle(sh, synth.weights(sh, seed=3))
    T = 0.9
    prompt = [3, 1, 4, 1, 5, 9, 2, 6]
    parents = np.array([-1, 0, 0, 1], dtype=np.int64)
    base = orc.new_seq(cap=32)
    base.commit(prompt[:-1])
    l0 = _copy(orc, base).step(prompt[-1])
    p0 = _softmax(np.asarray(l0, dtype=np.float32), T)
    p1 = np.zeros((16, 16))
    for a in range(16):
        s = _copy(orc, base)
        s.step(prompt[-1])
        p1[a] = _softmax(np.asarray(s.step(a), dtype=np.float32), T)
    joint = (p0[:, None] * p1).reshape(-1)

    counts = np.zeros(256, dtype=np.int64)
    n_seeds = 2000
    for sd in range(n_seeds):
        smp = oracle.Sampling(T, 1000 + sd)
        toks, _ = _rounds(orc, prompt[:-1], prompt[-1], 2,
                          lambda seq, root, par, r: synth.tree_tokens(par, 16, sd * 7 + r, root),
                          parents, smp, seq=_clone(orc, base))
        counts[toks[0] * 16 + toks[1]] += 1
    # pool cells with small expectation into one bin
    exp = n_seeds * joint
    big = exp >= 5
    obs = np.append(counts[big], counts[~big].sum())
    ex = np.append(exp[big], exp[~big].sum())
    p = stats.chisquare(obs, ex).pvalue
    assert p > 1e-3, p
