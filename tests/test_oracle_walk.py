"""Pins of the accept walk and of whole greedy rounds in the oracle.

"Drafters and tree verify", The round: verify reads the model's token at
every node; accept walks from the root, taking the model's token and moving
to the child that carries it, stopping where none does and keeping the
model's token there (so a round yields at least one token); commit keeps the
accepted path.  "Exactness", The promise: the emitted text equals plain greedy
decoding for any drafter, including one wrong on purpose on every token.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _all_parent_arrays(n):
    for rest in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(rest)


def _walk_by_definition(parents, tokens, argmax):
    """The accepted path is the deepest node all of whose edges p->c carry
    token[c] == argmax[p]; siblings carry distinct tokens, so it is unique."""
    n = len(parents)
    ok = [False] * n
    ok[0] = True
    depth = [0] * n
    for i in range(1, n):
        p = parents[i]
        ok[i] = ok[p] and tokens[i] == argmax[p]
        depth[i] = depth[p] + 1
    best = max((i for i in range(n) if ok[i]), key=lambda i: depth[i])
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = parents[j]
    path.reverse()
    emitted = [tokens[i] for i in path[1:]] + [argmax[best]]
    return path, emitted


def test_walk_brute_force_all_tiny_trees():
    count = 0
    for n in range(1, 6):
        for parents in _all_parent_arrays(n):
            kids = {}
            for i in range(1, n):
                kids.setdefault(parents[i], []).append(i)
            # every token assignment over {0,1,2} with distinct siblings
            for tok in itertools.product(range(3), repeat=n - 1):
                tokens = [9] + list(tok)
                if any(len({tokens[c] for c in cs}) != len(cs) for cs in kids.values()):
                    continue
                for am in itertools.product(range(3), repeat=n) if n <= 4 else \
                        [tuple(np.random.default_rng(count).integers(0, 3, n))]:
                    got = oracle.accept_walk(parents, tokens, am)
                    want = _walk_by_definition(parents, tokens, list(am))
                    assert got == (want[0], want[1]), (parents, tokens, am)
                    assert len(got[1]) >= 1
                    count += 1
    assert count > 5000


def _greedy_reference(orc, prompt, first, k):
    s = orc.new_seq(cap=256)
    s.commit(prompt)
    return oracle.greedy(s, first, k)[0]


def _run_rounds(orc, prompt, first, n_rounds, drafter, parents):
    """Greedy rounds in the oracle; returns every emitted token."""
    seq = orc.new_seq(cap=256)
    seq.commit(prompt)
    root = first
    out, per_round = [], []
    for r in range(n_rounds):
        tokens = drafter(seq, root, parents, r)
        logits = orc.tree_scores(seq, parents, tokens)
        am, _ = oracle.tree_decisions(logits, parents, tokens, seq.history)
        path, emitted = oracle.accept_walk(parents, tokens, am)
        seq.commit([int(tokens[i]) for i in path])
        out += emitted
        per_round.append(len(emitted))
        root = emitted[-1]
    return out, per_round


@pytest.fixture(scope="module")
def c0():
    return oracle.Oracle(synth.C0, synth.weights(synth.C0, seed=0))


def test_rounds_with_greedy_drafter_write_greedy_text(c0):
    prompt = synth.uniform_ids(64, synth.C0.vocab, 1)
    parents = synth.c0_tree()
    spine = synth.spine_nodes(parents)
    rng = np.random.default_rng(7)

    def drafter(seq, root, parents, r):
        # the oracle's own greedy continuation, kept with probability 0.7 a depth
        s = orc_copy(seq)
        cont = oracle.greedy(s, root, len(spine) - 1)[0]
        forced = {}
        for d, node in enumerate(spine[1:]):
            if rng.random() < 0.7:
                forced[node] = cont[d]
            else:
                break
        return synth.tree_tokens(parents, synth.C0.vocab, 100 + r, root, forced)

    def orc_copy(seq):
        s = c0.new_seq(cap=seq.cap)
        s.commit(seq.history)
        return s

    got, per_round = _run_rounds(c0, prompt[:-1], int(prompt[-1]), 8, drafter, parents)
    want = _greedy_reference(c0, prompt[:-1], int(prompt[-1]), len(got))
    assert got == want
    assert max(per_round) > 1          # the drafter was right sometimes


def test_rounds_with_wrong_drafter_write_one_token_each(c0):
    prompt = synth.uniform_ids(40, synth.C0.vocab, 2)
    parents = synth.c0_tree()

    def drafter(seq, root, parents, r):
        # every draft token differs from the model's own choice at its
        # parent; nodes are fixed in index order, so a parent's path is final
        # when its children are chosen
        s = c0.new_seq(cap=seq.cap)
        s.commit(seq.history)
        toks = synth.tree_tokens(parents, synth.C0.vocab, 200 + r, root)
        for i in range(1, len(parents)):
            p = int(parents[i])
            logits = c0.tree_scores(s, parents, toks, rows_wanted=[p])
            prior = s.history + oracle.path_tokens(parents, toks, p)
            am_p = oracle.top2(oracle.apply_modifiers(logits[p], prior, None))[0]
            sib = {int(toks[j]) for j in range(1, i) if parents[j] == p}
            t = int(toks[i])
            while t == am_p or t in sib:
                t = (t + 1) % synth.C0.vocab
            toks[i] = t
        return toks

    got, per_round = _run_rounds(c0, prompt[:-1], int(prompt[-1]), 6, drafter, parents)
    assert per_round == [1] * 6
    want = _greedy_reference(c0, prompt[:-1], int(prompt[-1]), 6)
    assert got == want
