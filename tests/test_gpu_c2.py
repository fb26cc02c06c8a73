"""The 64-layer stack at full size (44 GB of bf16 weights) on MI355X: sampled
rows of verifies at 1k and 8k context against the oracle, commits, and the
joint verify of two requests with score modifiers and a wrong drafter.

The oracle steps only the sampled rows and their ancestors (each step reads
the whole stack from host memory).  Every layer's cache holds synthetic
N(0,1) rows, so neither side needs a prefill.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

SHAPE = synth.C2
CAP = 8192 + 40


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def c2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import workloads
    _say("c2 build (64 layers, weights drawn on the device)")
    wl = workloads.build(SHAPE, max_ctx=CAP, max_req=2, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(SHAPE, wl.host_weights)
    ex = oracle.Oracle(SHAPE, wl.host_weights, exact=True)
    yield wl, orc, ex
    wl.tv.close()
    del wl, orc, ex
    gc.collect()
    torch.cuda.empty_cache()


def _context(wl, req, ctx, kv_seed, hist_seed):
    import workloads
    kv = synth.kv_cache(SHAPE, ctx, seed=kv_seed, cap=ctx)
    hist = synth.uniform_ids(ctx, SHAPE.vocab, hist_seed)
    workloads.load_context(wl, req, ctx, kv_seed, history=hist, src_kv={k: v.cuda() for k, v in kv.items()})
    return kv, hist


def _shallow_leaf(parents):
    """The branch leaf (a node off the spine) nearest the root."""
    spine = set(synth.spine_nodes(parents))
    depth = oracle.node_depths(parents)
    return min((depth[i], i) for i in range(len(parents)) if i not in spine)[1]


def _check_sampled(orc, ex, kv, ctx, hist, parents, tokens, sample, gl, am, gap, what, mods=None):
    """The sampled rows (and the ancestors they need) against the oracle's
    rounded and unrounded runs, through check_rows on the sub-tree."""
    from test_gpu_parity import check_rows
    rows = orc.tree_scores(orc.new_seq(cap=CAP, kv=kv, ctx_len=ctx, history=hist), parents, tokens,
                           rows_wanted=sample)
    rows_ex = ex.tree_scores(ex.new_seq(cap=CAP, kv=kv, ctx_len=ctx, history=hist), parents, tokens,
                             rows_wanted=sample)
    need = sorted(i for i in range(len(parents)) if not np.isnan(rows[i, 0]))
    idx = {i: j for j, i in enumerate(need)}
    sub_parents = [-1 if parents[i] < 0 else idx[int(parents[i])] for i in need]
    sub_tokens = [int(tokens[i]) for i in need]
    check_rows(gl[need], am[need], gap[need], rows[need], sub_parents, sub_tokens, hist, mods=mods,
               what=what, orc_exact=rows_ex[need])
    return need


@pytest.mark.parametrize("ctx,n", [(1024, 32), (8192, 32)])
def test_c2_sampled_rows_and_commit(c2, ctx, n):
    wl, orc, ex = c2
    _say(f"c2 verify n={n} ctx={ctx}")
    kv, hist = _context(wl, 0, ctx, 3, 30)
    parents = synth.spine_tree(n, 4)
    tokens = synth.tree_tokens(parents, SHAPE.vocab, 8, root_token=int(hist[-1]))
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    gl = wl.logits[:n].cpu().numpy().astype(np.float64)
    # a fixed verify is bitwise repeatable
    am2, _ = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    assert np.array_equal(gl, wl.logits[:n].cpu().numpy().astype(np.float64)) and np.array_equal(am, am2)
    # the tree's own KV rows as the verify wrote them (slot ctx + i), before the commit moves them
    rows_k = {l: wl.kv[0][(l, "k")][:, ctx:ctx + n].clone() for l in (0, 31, 63)}
    spine = synth.spine_nodes(parents)
    sample = [0, spine[1], _shallow_leaf(parents)]
    _say(f"c2 oracle rows {sample}")
    _check_sampled(orc, ex, kv, ctx, hist, parents, tokens, sample, gl, am, gap, f"c2 n={n} ctx={ctx} sampled")
    # commit a three-node path of the spine: the cache rows are gathered bit for bit
    path = spine[:3]
    wl.tv.commit(0, path)
    assert wl.tv.ctx_len(0) == ctx + len(path)
    torch.cuda.synchronize()
    for l, before in rows_k.items():
        after = wl.kv[0][(l, "k")][:, ctx:ctx + len(path)]
        assert torch.equal(after, before[:, path]), l


def test_c4_joint_64_layers(c2):
    """Two requests in one pass on the 64-layer stack (16 rows each, contexts
    1024 and 8192), score modifiers on every row ("Exactness", The promise;
    Parallel requests: a request's rows equal its alone verify) and a
    wrong-on-purpose drafter (one token per round, the oracle's token)."""
    wl, orc, ex = c2
    ctxs = (1024, 8192)
    ctx_state = []
    for r, ctx in enumerate(ctxs):
        kv, hist = _context(wl, r, ctx, 40 + r, 50 + r)
        mods = synth.modifiers(SHAPE.vocab, seed=7 + r)
        wl.tv.set_modifiers(r, mods.rep_penalty, mods.bias_ids, mods.bias_vals, mods.allow_bits)
        ctx_state.append((kv, hist, mods))
    roots = [int(ctx_state[r][1][-1]) for r in range(2)]
    try:
        for rnd in range(2):
            trees = []
            for r in range(2):
                parents = synth.spine_tree(16, 60 + r + rnd)
                tokens = synth.tree_tokens(parents, SHAPE.vocab, 70 + r + rnd, root_token=roots[r])
                # wrong on purpose: the root's children never carry the model's token
                am, _ = wl.tv.verify_tree(r, parents, tokens)
                for i in range(1, 16):
                    if parents[i] == 0 and tokens[i] == am[0]:
                        tokens[i] = (int(am[0]) + 1 + i) % SHAPE.vocab
                trees.append((parents, tokens))
            _say("c4 64 layers round", rnd)
            am_j, gap_j = wl.tv.verify_trees([0, 1], [t[0] for t in trees], [t[1] for t in trees],
                                             logits=wl.logits)
            joint = wl.logits[:32].clone()
            for r in range(2):
                parents, tokens = trees[r]
                kv, hist, mods = ctx_state[r]
                am_a, gap_a = wl.tv.verify_tree(r, parents, tokens, logits=wl.logits)
                assert torch.equal(wl.logits[:16], joint[16 * r:16 * r + 16]), "joint != alone"
                np.testing.assert_array_equal(am_a, am_j[16 * r:16 * r + 16])
                np.testing.assert_array_equal(gap_a, gap_j[16 * r:16 * r + 16])
                gl = joint[16 * r:16 * r + 16].cpu().numpy().astype(np.float64)
                if rnd == 0:
                    sample = [0, 1, _shallow_leaf(parents)]
                    _say(f"c4 64 layers oracle rows {sample} of request {r} (ctx {ctxs[r]})")
                    _check_sampled(orc, ex, kv, ctxs[r], hist, parents, tokens, sample, gl, am_a, gap_a,
                                   f"c4 64 layers req {r} ctx {ctxs[r]}", mods=mods)
                path, emitted = oracle.accept_walk(parents, tokens, am_a)
                assert len(emitted) == 1 and path == [0]
                wl.tv.commit(r, path)
                roots[r] = emitted[0]
    finally:
        for r in range(2):
            wl.tv.set_modifiers(r, 1.0)
