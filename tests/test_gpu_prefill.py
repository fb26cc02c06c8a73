"""Dense (MFMA) prefill on the chunk grid (MI355X only).

"Exactness", Caches: cache snapshots sit on chunk-grid boundaries, and a
request restored from one continues its prompt on those same boundaries, so
its arithmetic, and hence every bit of its output, matches a prefill that
started from nothing.

* The last row's token and the cache rows a dense prefill leaves agree with
  the oracle's sequential decode of the prompt (tokens up to near ties; the
  rows through the verify that reads them, within the logit tolerance).
* A prompt prefilled in two calls that split on a grid point, and a request
  resumed from a snapshot of the cache rows at a grid point, equal the cold
  prefill bit for bit (cache rows, last token, and the logits of a verify
  that follows).
* The dense and the chained (32-row) prefill continue with the same tokens
  up to near ties.
* Recurrent layers (plain gated and delta rule) take the chunk as chains of
  32 rows: the same checks, states included.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

LOGIT_ATOL = 2e-2


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def c0():
    _gpu()
    import workloads
    wl = workloads.build(synth.C0, max_ctx=512, max_req=3, weight_device="cuda", host_copy=True)
    return wl, oracle.Oracle(synth.C0, wl.host_weights)


def _kv(wl, req, n):
    return {k: v[:, :n].clone() for k, v in wl.kv[req].items()}


@pytest.mark.parametrize("n,chunk", [(200, 64), (37, 32), (300, 128), (64, 64)])
def test_c0_dense_prefill_against_oracle(c0, n, chunk):
    wl, orc = c0
    prompt = synth.uniform_ids(n + 1, synth.C0.vocab, 40 + n)
    _say("c0 dense prefill", n, chunk)
    wl.tv.set_history(0, [], 0)
    first = wl.tv.prefill_dense(0, prompt[:-1], chunk=chunk)
    assert wl.tv.ctx_len(0) == n
    seq = orc.new_seq(cap=512)
    last = seq.commit(prompt[:-1])
    a, _, _, g = oracle.top2(last)
    assert first == a or g <= 1.0, (first, a, g)
    # cache rows: bf16 values within a few bf16 steps of the oracle's
    for (l, nm), t in wl.kv[0].items():
        got = t[:, :n].float().cpu().numpy().astype(np.float64)
        want = (seq.K if nm == "k" else seq.V)[l][:, :n]
        err = np.abs(got - want)
        tol = 2.0 ** -6 * np.maximum(1.0, np.abs(want))
        assert (err <= tol).mean() > 0.999 and err.max() < 0.1, (l, nm, float(err.max()))
    # a verify that reads those rows, against the oracle's tree rows
    parents = synth.c0_tree()
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 7, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    ol = orc.tree_scores(seq, parents, tokens)
    gl = wl.logits[:len(parents)].cpu().numpy().astype(np.float64)
    assert np.abs(gl - ol).max() <= LOGIT_ATOL, float(np.abs(gl - ol).max())
    oam, ogap = oracle.tree_decisions(ol, parents, tokens, seq.history)
    for i in range(len(parents)):
        assert am[i] == oam[i] or ogap[i] <= 1.0


def test_c0_dense_prefill_largest_chunk():
    """The largest chunk the library takes (2048 rows) and a ragged second
    chunk, against the oracle's sequential decode of 2100 tokens; a resume at
    the grid point 2048 equals the cold prefill bit for bit."""
    _gpu()
    import workloads
    wl = workloads.build(synth.C0, max_ctx=2200, max_req=2, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(synth.C0, wl.host_weights)
    n, chunk = 2100, 2048
    prompt = synth.uniform_ids(n + 1, synth.C0.vocab, 91)
    _say("c0 dense prefill", n, chunk)
    wl.tv.set_history(0, [], 0)
    first = wl.tv.prefill_dense(0, prompt[:-1], chunk=chunk)
    seq = orc.new_seq(cap=2200)
    last = seq.commit(prompt[:-1])
    a, _, _, g = oracle.top2(last)
    assert first == a or g <= 1.0, (first, a, g)
    for (l, nm), t in wl.kv[0].items():
        got = t[:, :n].float().cpu().numpy().astype(np.float64)
        want = (seq.K if nm == "k" else seq.V)[l][:, :n]
        err = np.abs(got - want)
        tol = 2.0 ** -6 * np.maximum(1.0, np.abs(want))
        assert (err <= tol).mean() > 0.999 and err.max() < 0.1, (l, nm, float(err.max()))
    parents = synth.random_tree(32, 5)
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 8, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    ol = orc.tree_scores(seq, parents, tokens)
    gl = wl.logits[:len(parents)].cpu().numpy().astype(np.float64)
    assert np.abs(gl - ol).max() <= LOGIT_ATOL, float(np.abs(gl - ol).max())
    oam, ogap = oracle.tree_decisions(ol, parents, tokens, seq.history)
    for i in range(len(parents)):
        assert am[i] == oam[i] or ogap[i] <= 1.0
    # resumed at the grid point from the cold rows
    for key, t in wl.kv[1].items():
        t.zero_()
        t[:, :chunk].copy_(wl.kv[0][key][:, :chunk])
    wl.tv.set_history(1, prompt[:chunk].tolist(), chunk)
    assert wl.tv.prefill_dense(1, prompt[chunk:n], chunk=chunk) == first
    for key, t in wl.kv[1].items():
        assert torch.equal(t[:, :n], wl.kv[0][key][:, :n]), key


def test_c0_resume_on_the_grid_is_bitwise_cold(c0):
    wl, _ = c0
    chunk, n = 64, 230
    prompt = synth.uniform_ids(n + 1, synth.C0.vocab, 77)
    _say("c0 resume on the grid")
    # cold
    wl.tv.set_history(0, [], 0)
    cold_first = wl.tv.prefill_dense(0, prompt[:-1], chunk=chunk)
    cold = _kv(wl, 0, n)
    # the same prompt in two calls split on a grid point
    wl.tv.set_history(1, [], 0)
    wl.tv.prefill_dense(1, prompt[:128], chunk=chunk)
    split_first = wl.tv.prefill_dense(1, prompt[128:n], chunk=chunk)
    assert split_first == cold_first
    for key, t in _kv(wl, 1, n).items():
        assert torch.equal(t, cold[key]), key
    # resumed from a snapshot of the rows at grid point 192
    for key, t in wl.kv[2].items():
        t.zero_()
        t[:, :192].copy_(cold[key][:, :192])
    wl.tv.set_history(2, prompt[:192].tolist(), 192)
    res_first = wl.tv.prefill_dense(2, prompt[192:n], chunk=chunk)
    assert res_first == cold_first
    for key, t in _kv(wl, 2, n).items():
        assert torch.equal(t, cold[key]), key
    # and the logits of a verify that follows
    parents = synth.random_tree(16, 3)
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 9, root_token=int(prompt[-1]))
    outs = []
    for r in (0, 2):
        wl.tv.verify_tree(r, parents, tokens, logits=wl.logits)
        outs.append(wl.logits[:16].clone())
    assert torch.equal(outs[0], outs[1])


def test_c0_dense_and_chained_prefill_agree(c0):
    wl, orc = c0
    n = 150
    prompt = synth.uniform_ids(n + 1, synth.C0.vocab, 91)
    wl.tv.set_history(0, [], 0)
    a = wl.tv.prefill_dense(0, prompt[:-1], chunk=64)
    wl.tv.set_history(1, [], 0)
    b = wl.tv.prefill(1, prompt[:-1])
    seq = orc.new_seq(cap=512)
    last = seq.commit(prompt[:-1])
    o, _, _, g = oracle.top2(last)
    assert (a == o or g <= 1.0) and (b == o or g <= 1.0)
    for key in wl.kv[0]:
        d = (wl.kv[0][key][:, :n].float() - wl.kv[1][key][:, :n].float()).abs().max().item()
        assert d < 0.1, (key, d)


def test_c0_dense_prefill_errors(c0):
    from greedy_draft_tree_amd import TVError, TV_EINVAL, TV_ECAPACITY
    wl, _ = c0
    wl.tv.set_history(0, [], 0)
    for chunk in (16, 48, 4096):
        with pytest.raises(TVError) as e:
            wl.tv.prefill_dense(0, [1, 2, 3], chunk=chunk)
        assert e.value.code == TV_EINVAL
    with pytest.raises(TVError) as e:
        wl.tv.prefill_dense(0, [5] * 600, chunk=64)
    assert e.value.code == TV_ECAPACITY
    with pytest.raises(TVError):
        wl.tv.prefill_dense(0, [synth.C0.vocab], chunk=64)
    assert wl.tv.ctx_len(0) == 0


def test_c0_dense_prefill_sampled_last_token(c0):
    """A sampled request's prefill returns its draw at the index after the
    prompt, as plain sampled decoding does."""
    wl, orc = c0
    n = 90
    prompt = synth.uniform_ids(n, synth.C0.vocab, 13)
    smp = oracle.Sampling(0.9, 4242)
    wl.tv.set_history(0, [], 0)
    wl.tv.set_sampling(0, smp.temperature, smp.seed)
    try:
        got = wl.tv.prefill_dense(0, prompt, chunk=64)
    finally:
        wl.tv.set_sampling(0, 0.0)
    seq = orc.new_seq(cap=512)
    last = seq.commit(prompt)
    keys = oracle.sample_keys(oracle.apply_modifiers(last, seq.history, None), smp, n)
    a, l1, l2, _ = oracle.top2(keys)
    assert got == a or l1 - l2 <= 2 * LOGIT_ATOL / smp.temperature


HYBS = {k: synth.scaled(synth.C0, name, n_layer=4, kinds=[k, synth.ATTN, k, k])
        for k, name in ((synth.RECUR, "c0_hybrid_pf"), (synth.DELTA, "c0_delta_pf"))}


@pytest.mark.parametrize("kind", [synth.RECUR, synth.DELTA], ids=["gated", "delta"])
def test_hybrid_dense_prefill(kind):
    """Recurrent layers in the dense prefill (chains of 32 rows through the
    tree read-out, each committed): against the oracle's sequential decode
    (last token, states, a following verify), and a resume on the grid equal
    to the cold prefill bit for bit (states and cache rows)."""
    _gpu()
    import workloads
    shape = HYBS[kind]
    wl = workloads.build(shape, max_ctx=256, max_req=2, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(shape, wl.host_weights)
    s0 = synth.state0(shape, seed=6)
    n, chunk = 150, 64
    prompt = synth.uniform_ids(n + 1, shape.vocab, 21)
    _say("hybrid dense prefill", shape.name)
    for r in range(2):
        for l, t in wl.states[r].items():
            t.copy_(s0[l].cuda())
    torch.cuda.synchronize()
    wl.tv.set_history(0, [], 0)
    first = wl.tv.prefill_dense(0, prompt[:-1], chunk=chunk)
    seq = orc.new_seq(cap=256, s0=s0)
    last = seq.commit(prompt[:-1])
    a, _, _, g = oracle.top2(last)
    assert first == a or g <= 1.0, (first, a, g)
    torch.cuda.synchronize()
    for l, t in wl.states[0].items():
        got = t.cpu().numpy().astype(np.float64)
        err = np.abs(got - seq.S[l]).max()
        print(f"[{shape.name} prefill state {l}] max|dS| {err:.3g}", flush=True)
        assert err <= 2e-2 * max(1.0, np.abs(seq.S[l]).max()), (l, err)
    cold_states = {l: t.clone() for l, t in wl.states[0].items()}
    cold_kv = _kv(wl, 0, n)
    parents = synth.c0_tree()
    tokens = synth.tree_tokens(parents, shape.vocab, 7, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    ol = orc.tree_scores(seq, parents, tokens)
    gl = wl.logits[:len(parents)].cpu().numpy().astype(np.float64)
    assert np.abs(gl - ol).max() <= LOGIT_ATOL, float(np.abs(gl - ol).max())
    cold_logits = wl.logits[:len(parents)].clone()
    # resumed on the grid: the first 128 rows, then the rest
    wl.tv.set_history(1, [], 0)
    wl.tv.prefill_dense(1, prompt[:128], chunk=chunk)
    res_first = wl.tv.prefill_dense(1, prompt[128:n], chunk=chunk)
    assert res_first == first
    torch.cuda.synchronize()
    for l, t in wl.states[1].items():
        assert torch.equal(t, cold_states[l]), l
    for key, t in _kv(wl, 1, n).items():
        assert torch.equal(t, cold_kv[key]), key
    wl.tv.verify_tree(1, parents, tokens, logits=wl.logits)
    assert torch.equal(wl.logits[:len(parents)], cold_logits)


HYBW = {k: synth.scaled(synth.C1, name, n_layer=4, kinds=[k, synth.ATTN, k, k])
        for k, name in ((synth.RECUR, "c3_layers4_pf"), (synth.DELTA, "c3d_layers4_pf"))}


@pytest.mark.parametrize("kind", [synth.RECUR, synth.DELTA], ids=["gated", "delta"])
def test_hybrid_full_width_dense_prefill(kind):
    """Recurrent layers at full width (40 heads x 128 x 128 fp32 states,
    hidden 5120) in the dense prefill: 70 prompt rows in chunks of 64 (chains
    of 32, 32 and 6 rows) against the oracle's sequential decode (states, last
    token, a following verify at the oracle's bf16-drift tolerance)."""
    _gpu()
    import workloads
    from test_gpu_parity import check_rows
    shape = HYBW[kind]
    wl = workloads.build(shape, max_ctx=128, max_req=1, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(shape, wl.host_weights)
    s0 = synth.state0(shape, seed=6)
    for l, t in wl.states[0].items():
        t.copy_(s0[l].cuda())
    torch.cuda.synchronize()
    n = 70
    prompt = synth.uniform_ids(n + 1, shape.vocab, 23)
    _say("full-width hybrid dense prefill", shape.name, n)
    wl.tv.set_history(0, [], 0)
    first = wl.tv.prefill_dense(0, prompt[:-1], chunk=64)
    seq = orc.new_seq(cap=128, s0=s0)
    last = seq.commit(prompt[:-1])
    a, _, _, g = oracle.top2(last)
    assert first == a or g <= 2.0, (first, a, g)
    torch.cuda.synchronize()
    for l, t in wl.states[0].items():
        got = t.cpu().numpy().astype(np.float64)
        err = np.abs(got - seq.S[l]).max()
        print(f"[{shape.name} prefill state {l}] max|dS| {err:.3g}", flush=True)
        assert err <= 2e-2 * max(1.0, np.abs(seq.S[l]).max()), (l, err)
    parents = synth.spine_tree(8, 2)
    tokens = synth.tree_tokens(parents, shape.vocab, 3, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    ol = orc.tree_scores(seq, parents, tokens)
    ex = oracle.Oracle(shape, wl.host_weights, exact=True)
    es = ex.new_seq(cap=128, s0=s0)
    es.commit(prompt[:-1])
    oe = ex.tree_scores(es, parents, tokens)
    check_rows(wl.logits[:8].cpu().numpy(), am, gap, ol, parents, tokens, seq.history,
               what=f"{shape.name} after dense prefill", orc_exact=oe)


def test_c1_width_dense_prefill():
    """Full width (hidden 5120, 40 q heads, ffn 17408, the fp32 head): 96
    prompt rows in chunks of 64 against the oracle, then a verify."""
    _gpu()
    import workloads
    wl = workloads.build(synth.C1, max_ctx=256, max_req=1, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(synth.C1, wl.host_weights)
    n = 96
    prompt = synth.uniform_ids(n + 1, synth.C1.vocab, 5)
    _say("c1 width dense prefill", n)
    wl.tv.set_history(0, [], 0)
    first = wl.tv.prefill_dense(0, prompt[:-1], chunk=64)
    seq = orc.new_seq(cap=256)
    last = seq.commit(prompt[:-1])
    a, _, _, g = oracle.top2(last)
    assert first == a or g <= 2.0, (first, a, g)
    parents = synth.spine_tree(8, 2)
    tokens = synth.tree_tokens(parents, synth.C1.vocab, 3, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    ol = orc.tree_scores(seq, parents, tokens)
    gl = wl.logits[:8].cpu().numpy().astype(np.float64)
    err = np.abs(gl - ol).max()
    print(f"[c1 dense prefill] verify max|dlogit| {err:.4g}", flush=True)
    assert err <= 0.1, err


def test_full_width_prefill_chunk_size_is_bitwise():
    """A one-layer full-width gated-recurrence model (hidden 5120, ffn 17408)
    prefilled with chunks of 2048 rows (the stacked q/k/v projection and
    gate/up with SwiGLU on the 256 x 256 tiles) and with chunks of 64 (every
    projection on the 32-row-group kernel): recurrent layers take their rows
    as chains of 32 in order whatever the chunk, so the last token and the
    state after the prompt agree bit for bit."""
    _gpu()
    import workloads
    shape = synth.scaled(synth.C1, "c3_layer1_pf", n_layer=1, kinds=[synth.RECUR])
    wl = workloads.build(shape, max_ctx=2112, max_req=2, weight_device="cuda", host_copy=False)
    s0 = synth.state0(shape, seed=8)
    for r in (0, 1):
        for l, t in wl.states[r].items():
            t.copy_(s0[l].cuda())
    torch.cuda.synchronize()
    n = 2100
    prompt = synth.uniform_ids(n, shape.vocab, 29)
    _say("full-width prefill, chunk 2048 vs 64", n)
    firsts = []
    for r, chunk in ((0, 2048), (1, 64)):
        wl.tv.set_history(r, [], 0)
        firsts.append(wl.tv.prefill_dense(r, prompt, chunk=chunk))
    torch.cuda.synchronize()
    assert firsts[0] == firsts[1], firsts
    for l in wl.states[0]:
        assert torch.equal(wl.states[0][l], wl.states[1][l]), l
