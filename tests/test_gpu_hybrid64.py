"""The 64-layer hybrid stacks at full size on MI355X: 48 recurrent layers
(plain gated recurrence, or the gated delta rule) and 16 attention layers,
hidden 5120, 40 heads of 128 x 128 fp32 state ("Drafters and tree verify",
Tree verify through recurrent layers: the state advances separately along
each root-to-node path, and a commit keeps only the accepted path's state).

A 16-node tree at 1k context: sampled rows against the oracle (rounded and
unrounded runs), then a commit of a three-node path, and the committed
states of three recurrent layers against the oracle's sequential steps of
the same tokens.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("shape", [synth.C3, synth.C3D], ids=["gated", "delta"])
def test_hybrid64_tree_commit_states(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import workloads
    from test_gpu_c2 import _shallow_leaf
    from test_gpu_parity import check_rows
    ctx, n = 1024, 16
    cap = ctx + 32
    _say(f"{shape.name} build (64 layers, 48 recurrent)")
    wl = workloads.build(shape, max_ctx=cap, max_req=1, weight_device="cuda", host_copy=True)
    try:
        orc = oracle.Oracle(shape, wl.host_weights)
        ex = oracle.Oracle(shape, wl.host_weights, exact=True)
        kv = synth.kv_cache(shape, ctx, seed=3, cap=ctx)
        s0 = synth.state0(shape, seed=6)
        hist = synth.uniform_ids(ctx, shape.vocab, 30)
        workloads.load_context(wl, 0, ctx, 3, history=hist, src_kv={k: v.cuda() for k, v in kv.items()},
                               src_states={l: v.cuda() for l, v in s0.items()})
        parents = synth.spine_tree(n, 4)
        tokens = synth.tree_tokens(parents, shape.vocab, 21, root_token=int(hist[-1]))
        _say(f"{shape.name} verify n={n}")
        am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
        gl = wl.logits[:n].cpu().numpy().astype(np.float64)
        spine = synth.spine_nodes(parents)
        sample = [0, spine[1], _shallow_leaf(parents)]
        _say(f"{shape.name} oracle rows {sample}")
        rows = orc.tree_scores(orc.new_seq(cap=cap, kv=kv, ctx_len=ctx, history=hist, s0=s0), parents, tokens,
                               rows_wanted=sample)
        rows_ex = ex.tree_scores(ex.new_seq(cap=cap, kv=kv, ctx_len=ctx, history=hist, s0=s0), parents, tokens,
                                 rows_wanted=sample)
        need = sorted(i for i in range(n) if not np.isnan(rows[i, 0]))
        idx = {i: j for j, i in enumerate(need)}
        sub_parents = [-1 if parents[i] < 0 else idx[int(parents[i])] for i in need]
        check_rows(gl[need], am[need], gap[need], rows[need], sub_parents, [int(tokens[i]) for i in need], hist,
                   what=f"{shape.name} n={n} sampled", orc_exact=rows_ex[need])
        # commit three spine nodes; the oracle steps the same tokens
        path = spine[:3]
        wl.tv.commit(0, path)
        assert wl.tv.ctx_len(0) == ctx + len(path)
        _say(f"{shape.name} oracle commit of {len(path)} tokens")
        seq = orc.new_seq(cap=cap, kv=kv, ctx_len=ctx, history=hist, s0=s0)
        seq.commit([int(tokens[i]) for i in path])
        seq_ex = ex.new_seq(cap=cap, kv=kv, ctx_len=ctx, history=hist, s0=s0)
        seq_ex.commit([int(tokens[i]) for i in path])
        torch.cuda.synchronize()
        recur = [l for l, k in enumerate(shape.kinds) if k != synth.ATTN]
        for l in (recur[0], recur[len(recur) // 2], recur[-1]):
            got = wl.states[0][l].cpu().numpy().astype(np.float64)
            want = seq.S[l]
            err = np.abs(got - want).max()
            # A deep layer's state is built from the bf16 residual stream of the
            # layers below it, so it carries their rounding drift.  The oracle's
            # own drift from its unrounded run (spread) measures what bf16
            # rounding does on this layer; the GPU and the oracle are two
            # computations with the same rounding points, each expected within
            # about that drift of the unrounded state, so they may differ by up
            # to twice it (triangle inequality).  Floor: 2e-2 of the state's scale.
            spread = np.abs(want - seq_ex.S[l]).max()
            to_exact = np.abs(got - seq_ex.S[l]).max()
            tol = 2.0 * max(2e-2 * max(1.0, np.abs(want).max()), spread)
            print(f"[{shape.name} state layer {l}] max|dS| {err:.3g} (to the unrounded state {to_exact:.3g}) "
                  f"max|S| {np.abs(want).max():.3g} oracle spread {spread:.3g} tol {tol:.3g}", flush=True)
            assert err <= tol, (l, err, tol)
    finally:
        wl.tv.close()
        del wl
        gc.collect()
        torch.cuda.empty_cache()
