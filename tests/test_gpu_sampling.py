"""Parity of the sampled tree verify with the CPU oracle (MI355X only).

"Exactness", Sampling and "Drafters and tree verify", Sampling: a sampled
request draws the target's own token at every node (the argmax of the
modified scores over T plus Gumbel noise keyed by (seed, t)), and a drafted
token survives exactly while the draw lands on it, so a seed's text is the
same for any drafter.

Bars:
  * the GPU's draw and key gap at every row are those the oracle takes from
    the GPU's own fp32 logits (bit for bit; the noise is fp64 logs rounded to
    fp32 on both sides, so a key may differ by one fp32 ulp where the two
    fp64 libraries round differently: a draw may then differ only where the
    two best keys are that close);
  * against the oracle's own logits, a draw may differ only where the
    oracle's two best keys lie within what the logit tolerance, divided by T,
    can reorder;
  * texts of one seed are identical, token for token, for every drafter,
    and equal the oracle's plain sampled decoding up to such a near tie.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

LOGIT_ATOL = 2e-2
OWN_GAP_ATOL = 1e-3     # bf16 ulps: one fp32 ulp of a key is about 2^-16 of them


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print("[case]", *a, flush=True)


def _key_gap_abs(keys):
    a, l1, l2, _ = oracle.top2(keys)
    return l1 - l2


def check_sampled(gpu_logits, draw, gap, orc_logits, parents, tokens, history, ctx_len, smp, mods=None,
                  what="", orc_exact=None):
    n = len(parents)
    gl = gpu_logits[:n].astype(np.float64)
    diff = np.abs(gl - orc_logits[:n])
    tol = np.full(n, LOGIT_ATOL)
    if orc_exact is not None:
        tol = np.maximum(tol, np.abs(orc_logits[:n] - orc_exact[:n]).max(axis=1))
    print(f"[{what}] max|dlogit| {diff.max():.4g}", flush=True)
    assert (diff.max(axis=1) <= tol).all(), f"{what}: logits over tolerance"
    # the GPU's decisions are the oracle's on the GPU's own logits
    own_am, own_gap = oracle.sampled_tree_decisions(gl, parents, tokens, history, ctx_len, smp, mods)
    for i in range(n):
        if draw[i] != own_am[i]:
            assert own_gap[i] <= OWN_GAP_ATOL, f"{what}: row {i} draw {draw[i]} vs own {own_am[i]}"
    fin = np.isfinite(own_gap)
    np.testing.assert_allclose(gap[:n][fin], own_gap[fin], rtol=0, atol=OWN_GAP_ATOL,
                               err_msg=f"{what}: key gap vs own logits")
    assert np.array_equal(np.isfinite(gap[:n]), fin)
    # against the oracle's logits: flips only where the logit tolerance can reorder the keys
    am, ogap = oracle.sampled_tree_decisions(orc_logits[:n], parents, tokens, history, ctx_len, smp, mods)
    dep = oracle.node_depths(parents)
    flips = 0
    for i in range(n):
        if draw[i] == am[i]:
            continue
        prior = list(history) + oracle.path_tokens(parents, tokens, i)
        keys = oracle.sample_keys(oracle.apply_modifiers(orc_logits[i], prior, mods), smp,
                                  ctx_len + dep[i] + 1)
        assert _key_gap_abs(keys) <= 2 * tol[i] / smp.temperature + 1e-5, \
            f"{what}: row {i} draw {draw[i]} vs oracle {am[i]} (key gap {ogap[i]:.3f} ulp)"
        flips += 1
    if flips:
        print(f"[{what}] draws that differ at near ties: {flips}", flush=True)
    return flips


# ------------------------------------------------------------------ C0

@pytest.fixture(scope="module")
def c0():
    _gpu()
    import workloads
    wl = workloads.build(synth.C0, max_ctx=512, max_req=2, weight_device="cuda", host_copy=True)
    return wl, oracle.Oracle(synth.C0, wl.host_weights)


@pytest.mark.parametrize("T", [0.8, 50.0])
def test_c0_sampled_prefill_and_tree_rows(c0, T):
    wl, orc = c0
    smp = oracle.Sampling(T, 0x5EED0000 + int(T))
    prompt = synth.uniform_ids(64, synth.C0.vocab, 1)
    _say("c0 sampled prefill 63, T", T)
    wl.tv.set_history(0, [], 0)
    wl.tv.set_sampling(0, T, smp.seed)
    try:
        first = wl.tv.prefill(0, prompt[:-1])
        seq = orc.new_seq(cap=512)
        last = seq.commit(prompt[:-1])
        # the prefill's last row draws index 63
        keys = oracle.sample_keys(oracle.apply_modifiers(last, seq.history, None), smp, 63)
        a, _, _, g = oracle.top2(keys)
        assert first == a or _key_gap_abs(keys) <= 2 * LOGIT_ATOL / T
        for seed, parents in [(2, synth.c0_tree()), (3, synth.spine_tree(32, 3)), (4, synth.chain_tree(1)),
                              (5, synth.bush_tree(17)), (6, synth.random_tree(29, 6))]:
            tokens = synth.tree_tokens(parents, synth.C0.vocab, seed, root_token=int(prompt[-1]))
            _say("c0 sampled tree", seed, len(parents), "T", T)
            draw, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
            gl = wl.logits[:len(parents)].cpu().numpy()
            ol = orc.tree_scores(seq, parents, tokens)
            check_sampled(gl, draw, gap, ol, parents, tokens, seq.history, seq.ctx_len, smp,
                          what=f"c0 sampled tree {seed} T={T}")
    finally:
        wl.tv.set_sampling(0, 0.0)


def _gpu_text(wl, req, prompt, n_tokens, smp, drafter, mods=None):
    """Sampled rounds on the GPU (tv_round); returns (text, tokens per round)."""
    wl.tv.set_history(req, [], 0)
    if mods is not None:
        wl.tv.set_modifiers(req, mods.rep_penalty, mods.bias_ids, mods.bias_vals, mods.allow_bits)
    else:
        wl.tv.set_modifiers(req, 1.0)
    wl.tv.set_sampling(req, smp.temperature, smp.seed)
    try:
        wl.tv.prefill(req, prompt[:-1])
        root, out, per_round, r = int(prompt[-1]), [], [], 0
        while len(out) < n_tokens:
            parents, tokens = drafter(root, len(out), r)
            _, _, path, emitted = wl.tv.round(req, parents, tokens)
            out += list(emitted)
            per_round.append(len(emitted))
            root, r = int(emitted[-1]), r + 1
        return out[:n_tokens], per_round
    finally:
        wl.tv.set_sampling(req, 0.0)
        wl.tv.set_modifiers(req, 1.0)


def _drafters(ref, vocab):
    """Drafters over the c0 tree: 'root' proposes nothing, 'right' the
    reference text's next tokens along the spine (kept with probability 0.7
    a depth), 'wrong' root children that all miss the next token, 'random'
    random tokens everywhere."""
    parents = synth.c0_tree()
    spine = synth.spine_nodes(parents)
    rng = np.random.default_rng(11)

    def root(root_tok, done, r):
        return [-1], [root_tok]

    def right(root_tok, done, r):
        forced = {}
        for d, node in enumerate(spine[1:]):
            if done + d >= len(ref) or rng.random() >= 0.7:
                break
            forced[node] = ref[done + d]
        return parents, synth.tree_tokens(parents, vocab, 900 + r, root_tok, forced)

    def wrong(root_tok, done, r):
        toks = synth.tree_tokens(parents, vocab, 950 + r, root_tok)
        nxt = ref[done] if done < len(ref) else -1
        kids = [i for i in range(1, len(parents)) if parents[i] == 0]
        used = {int(toks[i]) for i in kids}
        for i in kids:
            if toks[i] == nxt:
                t = (nxt + 1) % vocab
                while t in used:
                    t = (t + 1) % vocab
                toks[i] = t
                used.add(t)
        return parents, toks

    def rand(root_tok, done, r):
        return parents, synth.tree_tokens(parents, vocab, 990 + r, root_tok)

    return {"root": root, "right": right, "wrong": wrong, "random": rand}


@pytest.mark.parametrize("with_mods", [False, True])
def test_c0_sampled_text_same_for_every_drafter(c0, with_mods):
    wl, orc = c0
    smp = oracle.Sampling(0.9 if not with_mods else 1.4, 0xABCDEF0123 + with_mods)
    mods = synth.modifiers(synth.C0.vocab, seed=4, n_bias=32, penalty=1.3, allow_frac=0.4) \
        if with_mods else None
    prompt = synth.uniform_ids(48, synth.C0.vocab, 3)
    K = 24
    _say("c0 sampled text, root-only drafter, mods", with_mods)
    ref, per = _gpu_text(wl, 1, prompt, K, smp, _drafters([], synth.C0.vocab)["root"], mods)
    assert per == [1] * K
    d = _drafters(ref, synth.C0.vocab)
    for kind in ("right", "wrong", "random"):
        _say("c0 sampled text, drafter", kind)
        got, per = _gpu_text(wl, 1, prompt, K, smp, d[kind], mods)
        assert got == ref, kind
        if kind == "right":
            assert max(per) > 1
        if kind == "wrong":
            assert per == [1] * K
    # the oracle's plain sampled decoding writes the same text up to a near tie
    s = orc.new_seq(cap=512)
    s.commit(prompt[:-1])
    t = int(prompt[-1])
    for k in range(K):
        logits = s.step(t)
        keys = oracle.sample_keys(oracle.apply_modifiers(logits, s.history, mods), smp, s.ctx_len)
        a = oracle.top2(keys)[0]
        if a != ref[k]:
            assert _key_gap_abs(keys) <= 2 * LOGIT_ATOL / smp.temperature, (k, a, ref[k])
            print(f"[c0 text] near tie at token {k}; the rest follows the GPU's text", flush=True)
        t = ref[k]
    if with_mods:
        ids = np.asarray(ref)
        assert np.all((mods.allow_bits[ids // 32] >> (ids % 32).astype(np.uint32)) & 1)


def test_c0_temperature_zero_is_greedy_bitwise(c0):
    wl, _ = c0
    prompt = synth.uniform_ids(30, synth.C0.vocab, 8)
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, prompt[:-1])
    parents = synth.random_tree(32, 9)
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 10, root_token=int(prompt[-1]))
    am0, gap0 = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    l0 = wl.logits.clone()
    wl.tv.set_sampling(0, 0.7, 123)
    am1, gap1 = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    assert torch.equal(wl.logits, l0), "sampling must not touch the returned logits"
    assert not np.array_equal(am1, am0)
    wl.tv.set_sampling(0, 0.0, 123)
    am2, gap2 = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    np.testing.assert_array_equal(am2, am0)
    np.testing.assert_array_equal(gap2, gap0)


def test_c0_sampling_errors_leave_state(c0):
    from greedy_draft_tree_amd import TVError, TV_EINVAL
    wl, _ = c0
    wl.tv.set_sampling(0, 0.0)
    for T in (-0.5, float("nan"), float("inf")):
        with pytest.raises(TVError) as e:
            wl.tv.set_sampling(0, T, 1)
        assert e.value.code == TV_EINVAL
    with pytest.raises(TVError):
        wl.tv.set_sampling(7, 1.0, 1)
    prompt = synth.uniform_ids(20, synth.C0.vocab, 12)
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, prompt[:-1])
    parents = synth.c0_tree()
    tokens = synth.tree_tokens(parents, synth.C0.vocab, 13, root_token=int(prompt[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    # still greedy: every row's pick is the argmax of its own logits
    gl = wl.logits[:len(parents)].cpu().numpy()
    np.testing.assert_array_equal(am, np.argmax(gl, axis=1))


# ------------------------------------------------------------------ C1

@pytest.fixture(scope="module")
def c1():
    _gpu()
    import workloads
    wl = workloads.build(synth.C1, max_ctx=4096 + 64, max_req=2, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(synth.C1, wl.host_weights)
    orc.w_src = wl.host_weights
    return wl, orc


@pytest.mark.parametrize("n,ctx,T,with_mods", [(32, 1024, 0.7, False), (32, 1024, 50.0, False),
                                               (24, 3000, 1.1, True)])
def test_c1_sampled_tree_rows(c1, n, ctx, T, with_mods):
    import workloads
    wl, orc = c1
    _say("c1 sampled", n, ctx, T, with_mods)
    smp = oracle.Sampling(T, 0x1234567800000000 + n + ctx)
    kv = synth.kv_cache(synth.C1, ctx, seed=3, cap=ctx)
    hist = synth.uniform_ids(ctx, synth.C1.vocab, 30)
    workloads.load_context(wl, 0, ctx, 3, history=hist, src_kv={k: v.cuda() for k, v in kv.items()})
    mods = synth.modifiers(synth.C1.vocab, seed=21) if with_mods else None
    if mods is not None:
        wl.tv.set_modifiers(0, mods.rep_penalty, mods.bias_ids, mods.bias_vals, mods.allow_bits)
    wl.tv.set_sampling(0, T, smp.seed)
    try:
        parents = synth.spine_tree(n, 4)
        tokens = synth.tree_tokens(parents, synth.C1.vocab, 5 + n, root_token=int(hist[-1]))
        draw, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    finally:
        wl.tv.set_sampling(0, 0.0)
        wl.tv.set_modifiers(0, 1.0)
    gl = wl.logits[:n].cpu().numpy()
    seq = orc.new_seq(cap=ctx + 32, kv=kv, ctx_len=ctx, history=hist)
    ol = orc.tree_scores(seq, parents, tokens)
    ex = oracle.Oracle(synth.C1, orc.w_src, exact=True)
    oe = ex.tree_scores(ex.new_seq(cap=ctx + 32, kv=kv, ctx_len=ctx, history=hist), parents, tokens)
    check_sampled(gl, draw, gap, ol, parents, tokens, seq.history, ctx, smp, mods,
                  what=f"c1 sampled n={n} ctx={ctx} T={T}", orc_exact=oe)


def test_c1_joint_sampled_and_greedy_equal_alone(c1):
    """Two requests in one pass, one sampled with modifiers and one greedy
    ("Exactness", Parallel requests): each request's logits, picks and gaps
    equal its alone verify bit for bit, and the sampled rows' draws are the
    oracle's on the GPU's logits."""
    import workloads
    wl, orc = c1
    ctxs = (1024, 4096)
    smp = oracle.Sampling(0.9, 77)
    mods = synth.modifiers(synth.C1.vocab, seed=8)
    trees, hists = [], []
    for r, ctx in enumerate(ctxs):
        hist = synth.uniform_ids(ctx, synth.C1.vocab, 50 + r)
        workloads.load_context(wl, r, ctx, 40 + r, history=hist)
        parents = synth.spine_tree(16, 60 + r)
        trees.append((parents, synth.tree_tokens(parents, synth.C1.vocab, 70 + r, root_token=int(hist[-1]))))
        hists.append(hist)
    wl.tv.set_modifiers(0, mods.rep_penalty, mods.bias_ids, mods.bias_vals, mods.allow_bits)
    wl.tv.set_sampling(0, smp.temperature, smp.seed)
    try:
        _say("c4 joint sampled + greedy")
        am_j, gap_j = wl.tv.verify_trees([0, 1], [t[0] for t in trees], [t[1] for t in trees],
                                         logits=wl.logits)
        joint = wl.logits[:32].clone()
        for r in range(2):
            parents, tokens = trees[r]
            am_a, gap_a = wl.tv.verify_tree(r, parents, tokens, logits=wl.logits)
            assert torch.equal(wl.logits[:16], joint[16 * r:16 * r + 16]), "joint != alone"
            np.testing.assert_array_equal(am_a, am_j[16 * r:16 * r + 16])
            np.testing.assert_array_equal(gap_a, gap_j[16 * r:16 * r + 16])
            gl = joint[16 * r:16 * r + 16].cpu().numpy().astype(np.float64)
            if r == 0:
                own_am, own_gap = oracle.sampled_tree_decisions(gl, parents, tokens, list(hists[0]),
                                                                ctxs[0], smp, mods)
            else:
                own_am, own_gap = oracle.tree_decisions(gl, parents, tokens, list(hists[1]), None)
            bad = [i for i in range(16) if am_a[i] != own_am[i] and own_gap[i] > OWN_GAP_ATOL]
            assert not bad, (r, bad)
    finally:
        wl.tv.set_sampling(0, 0.0)
        wl.tv.set_modifiers(0, 1.0)
