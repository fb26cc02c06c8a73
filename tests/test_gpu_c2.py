"""The 64-layer stack at full size (44 GB of bf16 weights) on MI355X: sampled
rows of a 32-node verify at 1k context against the oracle, then a commit.

The oracle steps only the sampled rows and their ancestors (each step reads
the whole stack from host memory).  Every layer's cache holds 1024 synthetic
N(0,1) rows, so neither side needs a prefill.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def test_c2_sampled_rows_and_commit():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import workloads
    from test_gpu_parity import check_rows
    shape, ctx, n = synth.C2, 1024, 32
    print("[case] c2 build (64 layers, weights drawn on the device)", flush=True)
    wl = workloads.build(shape, max_ctx=ctx + 40, max_req=1, weight_device="cuda", host_copy=True)
    kv = synth.kv_cache(shape, ctx, seed=3, cap=ctx)
    hist = synth.uniform_ids(ctx, shape.vocab, 30)
    workloads.load_context(wl, 0, ctx, 3, history=hist, src_kv={k: v.cuda() for k, v in kv.items()})
    parents = synth.spine_tree(n, 4)
    tokens = synth.tree_tokens(parents, shape.vocab, 8, root_token=int(hist[-1]))
    print("[case] c2 verify n=32", flush=True)
    am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    gl = wl.logits[:n].cpu().numpy().astype(np.float64)
    # a fixed verify is bitwise repeatable
    am2, _ = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
    assert np.array_equal(gl, wl.logits[:n].cpu().numpy().astype(np.float64)) and np.array_equal(am, am2)
    spine = synth.spine_nodes(parents)
    leaf = n - 1
    sample = [0, spine[2], leaf]
    print(f"[case] c2 oracle rows {sample}", flush=True)
    orc = oracle.Oracle(shape, wl.host_weights)
    rows = orc.tree_scores(orc.new_seq(cap=ctx + 40, kv=kv, ctx_len=ctx, history=hist), parents, tokens,
                           rows_wanted=sample)
    ex = oracle.Oracle(shape, wl.host_weights, exact=True)
    rows_ex = ex.tree_scores(ex.new_seq(cap=ctx + 40, kv=kv, ctx_len=ctx, history=hist), parents, tokens,
                             rows_wanted=sample)
    need = sorted(i for i in range(n) if not np.isnan(rows[i, 0]))
    idx = {i: j for j, i in enumerate(need)}
    sub_parents = [-1 if parents[i] < 0 else idx[int(parents[i])] for i in need]
    sub_tokens = [int(tokens[i]) for i in need]
    check_rows(gl[need], am[need], gap[need], rows[need], sub_parents, sub_tokens, hist,
               what="c2 n=32 sampled", orc_exact=rows_ex[need])
    path, emitted = oracle.accept_walk(parents, tokens, am)
    wl.tv.commit(0, path)
    assert wl.tv.ctx_len(0) == ctx + len(path)
