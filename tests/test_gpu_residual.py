"""Residual tree sampling on the GPU against the oracle (MI355X only).

"Algorithm and correctness contract", Deterministic tree candidates and
residual verification.  Bars: with the same uniforms, the GPU's round (path
and emitted tokens) equals the oracle's residual walk on the GPU's own fp32
logits, except where a decision's margin (running sum against u times the
total, relative) is below 1e-9 (fp64 sums in another order); against the
oracle's own logits it may differ only where the logit tolerance can move
the decision (the round's margin below 0.05).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def c0():
    _gpu()
    import workloads
    wl = workloads.build(synth.C0, max_ctx=512, max_req=1, weight_device="cuda", host_copy=True)
    return wl, oracle.Oracle(synth.C0, wl.host_weights)


@pytest.mark.parametrize("T", [0.7, 1.0, 3.0])
def test_c0_residual_rounds(c0, T):
    wl, orc = c0
    prompt = synth.uniform_ids(60, synth.C0.vocab, 3)
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, prompt[:-1])
    seq = orc.new_seq(cap=512)
    seq.commit(prompt[:-1])
    rng = np.random.default_rng(int(T * 10))
    root = int(prompt[-1])
    same_as_oracle = 0
    for r in range(10):
        parents = synth.random_tree(int(rng.integers(1, 20)), 50 + r) if r % 3 else synth.c0_tree()
        tokens = synth.tree_tokens(parents, synth.C0.vocab, 60 + r, root_token=root)
        u = rng.random(32)
        _say("c0 residual round", T, r, len(parents))
        path, emitted = wl.tv.residual_round(0, parents, tokens, T, u, logits=wl.logits)
        gl = wl.logits[:len(parents)].cpu().numpy()
        opath, oemit, margin = oracle.residual_walk(gl, parents, tokens, seq.history, T, u)
        if margin > 1e-9:
            assert (path, emitted) == (opath, oemit), (r, path, opath, emitted, oemit)
        ol = orc.tree_scores(seq, parents, tokens)
        p2, e2, m2 = oracle.residual_walk(ol, parents, tokens, seq.history, T, u)
        if (p2, e2) == (path, emitted):
            same_as_oracle += 1
        else:
            assert m2 < 0.05, (r, m2)
        seq.commit([int(tokens[i]) for i in path])
        assert wl.tv.ctx_len(0) == seq.ctx_len
        root = emitted[-1]
    assert same_as_oracle >= 8


def test_c0_residual_accepts_the_first_child(c0):
    """A round whose first candidate is the model's near-certain token (a low
    temperature) accepts it: the decision that names candidate 0 is encoded
    as -1 in the row's record, the same value that marks a record empty, so
    completion must be read from the record's other field."""
    wl, orc = c0
    prompt = synth.uniform_ids(30, synth.C0.vocab, 12)
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, prompt[:-1])
    seq = orc.new_seq(cap=512)
    seq.commit(prompt[:-1])
    root = int(prompt[-1])
    g = int(wl.tv.verify_tree(0, [-1], [root], logits=wl.logits)[0][0])
    other = (g + 1) % synth.C0.vocab
    parents, tokens = [-1, 0, 0], [root, g, other]
    u = np.full(32, 0.01)   # accepted whenever p(g) > 0.01, certain for the argmax at T = 0.05
    _say("c0 residual accepts candidate 0")
    path, emitted = wl.tv.residual_round(0, parents, tokens, 0.05, u, logits=wl.logits)
    gl = wl.logits[:3].cpu().numpy()
    opath, oemit, margin = oracle.residual_walk(gl, parents, tokens, seq.history, 0.05, u)
    assert path[:2] == [0, 1] and (path, emitted) == (opath, oemit), (path, emitted, opath, oemit, margin)


def test_c0_residual_errors_leave_state(c0):
    from greedy_draft_tree_amd import TVError, TV_EINVAL
    wl, _ = c0
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, synth.uniform_ids(20, synth.C0.vocab, 4))
    n0 = wl.tv.ctx_len(0)
    parents = synth.c0_tree()
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 5, root_token=3)
    for T, u in ((0.0, np.full(8, 0.5)), (1.0, np.full(8, 1.0)), (1.0, np.full(8, -0.1))):
        with pytest.raises(TVError) as e:
            wl.tv.residual_round(0, parents, tokens, T, u)
        assert e.value.code == TV_EINVAL
    assert wl.tv.ctx_len(0) == n0


def test_c1_residual_round_full_vocab_with_modifiers():
    """Full vocabulary (151936 ids), score modifiers, and temperatures that
    put the residual draw anywhere in the vocabulary."""
    _gpu()
    import workloads
    wl = workloads.build(synth.C1, max_ctx=1024 + 64, max_req=1, weight_device="cuda", host_copy=True)
    ctx = 1024
    kv = synth.kv_cache(synth.C1, ctx, seed=3, cap=ctx)
    hist = synth.uniform_ids(ctx, synth.C1.vocab, 30)
    mods = synth.modifiers(synth.C1.vocab, seed=21)
    rng = np.random.default_rng(5)
    for T in (0.8, 40.0):
        for r in range(3):
            workloads.load_context(wl, 0, ctx, 3, history=hist, src_kv={k: v.cuda() for k, v in kv.items()})
            wl.tv.set_modifiers(0, mods.rep_penalty, mods.bias_ids, mods.bias_vals, mods.allow_bits)
            try:
                parents = synth.spine_tree(16, 7 + r)
                tokens = synth.tree_tokens(parents, synth.C1.vocab, 8 + r, root_token=int(hist[-1]))
                u = rng.random(32)
                _say("c1 residual", T, r)
                path, emitted = wl.tv.residual_round(0, parents, tokens, T, u, logits=wl.logits)
            finally:
                wl.tv.set_modifiers(0, 1.0)
            gl = wl.logits[:16].cpu().numpy()
            opath, oemit, margin = oracle.residual_walk(gl, parents, tokens, list(hist), T, u, mods)
            if margin > 1e-9:
                assert (path, emitted) == (opath, oemit), (T, r, path, opath, emitted, oemit)
            ids = np.asarray(emitted)
            assert np.all((mods.allow_bits[ids // 32] >> (ids % 32).astype(np.uint32)) & 1)
