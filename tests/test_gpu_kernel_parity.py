"""Kernel-level parity on identical inputs (MI355X only).

Each kernel of the pass besides the projections and the head (those are in
test_gpu_kernels.py) runs through its own C-ABI call on seeded synthetic
inputs, and its output is held against the oracle's own function on the
same inputs:

* tree attention + combine (tv_attention) against ``Oracle.attention`` on
  each node's cached context plus its ancestors-or-self;
* RoPE + KV write, which also finishes the QKV partial sums (tv_rope_kv),
  against ``Oracle.rope`` on the bf16-rounded sums;
* residual add + RMSNorm (tv_resid_norm) against ``oracle.rms_norm``;
* the recurrent tree read-out, plain gated and gated delta rule
  (tv_recur_tree), against ``Oracle.recurrent_token`` stepped along every
  root-to-node path, and the closed-form state commit (tv_recur_commit)
  against the oracle's state after the accepted path;
* the KV gather of the commit (tv_gather_kv) against a plain gather.

The bar for a bf16 output: it is the correctly rounded (nearest-even) bf16
value of the oracle's unrounded result, except where that result lies within
the kernel's fp32 error bound delta of a rounding midpoint, where either
neighbour passes; i.e. |gpu - exact| <= ulp(exact)/2 + delta everywhere.
delta is derived per element from the kernel's arithmetic (each docstring
below).  Integer and copy outputs are bit-exact.  The split-K partials are
dyadic (synth.dyadic_partials), so their fp32 sum is exact on both sides.
Shapes: the full-width layer (40 query / 8 KV heads of 128, hidden 5120) at
the contexts and row counts the benchmark runs, and the tiny model's heads
of 64, with ragged contexts (not a multiple of the 64-key chunk), one-row
trees and empty contexts.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24          # fp32 unit roundoff


def gamma(n):
    return n * U / (1 - n * U)


def _say(*a):
    print("[case]", *a, flush=True)


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(oracle.t2u16(t))


def check_rounded(gpu: np.ndarray, exact: np.ndarray, delta, what: str):
    """|gpu - exact| <= ulp_bf16(exact)/2 + delta everywhere; report how many
    outputs are exactly the correctly rounded value."""
    exact = np.asarray(exact, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    delta = np.broadcast_to(np.asarray(delta, dtype=np.float64), exact.shape)
    rounded = oracle.bf16_round(exact)
    err = np.abs(gpu - exact)
    lim = oracle.ulp_bf16(exact) / 2 + delta
    bad = err > lim
    frac = float((gpu == rounded).mean())
    print(f"[{what}] {exact.size} outputs, correctly rounded {frac:.6f}, "
          f"max err/ulp {float((err / oracle.ulp_bf16(exact)).max()):.3f}, "
          f"max delta/ulp {float((delta / oracle.ulp_bf16(exact)).max()):.3g}", flush=True)
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs beyond half an ulp + delta; first at "
                           f"{np.argwhere(bad)[0].tolist()}: gpu {gpu[bad][0]!r} exact {exact[bad][0]!r}")
    # outputs outside delta of a midpoint must be exactly the rounded value
    far = np.abs(np.abs(exact - rounded) - oracle.ulp_bf16(exact) / 2) > delta
    assert np.array_equal(gpu[far], rounded[far]), f"{what}: rounding differs away from a midpoint"
    return frac


def _tv(shape, max_ctx):
    from greedy_draft_tree_amd import TreeVerifier
    stream = torch.cuda.current_stream().cuda_stream
    return TreeVerifier.for_shape(shape, max_ctx=max_ctx, max_req=1, stream=stream)


FULL = synth.C1
TINY = synth.C0


@pytest.fixture(scope="module")
def tvs():
    _gpu()
    out = {FULL.name: _tv(FULL, 8192 + 64), TINY.name: _tv(TINY, 8192 + 64)}
    yield out
    for t in out.values():
        t.close()


def _ancestors(parents, t):
    out = []
    while t >= 0:
        out.append(t)
        t = int(parents[t])
    return out[::-1]


# ------------------------------------------------------------- attention

def _attention_delta(q, Kk, Vv, D, chunks_per_split, n_splits):
    """Bound of the kernel's fp32 error for one (node, head): score dot
    products on the matrix cores (bf16 products exact, fp32 sums of D
    terms: gamma_D sum|k q|), moved into the weights through the softmax
    (x2 for numerator and denominator), and the accumulation of P V: each
    64-key chunk adds 8 matrix instructions of 16 products (P split into
    bf16 high and low parts, |P - hi - lo| <= 2^-18 P), the chunks of a split
    are rescaled once each, and the combine adds up to 33 splits; exp2 and
    the final division add a few ulps.  delta = (2 scale gamma_D max_j
    sum|k_j q| + gamma_A + 2^-17) * sum_j p_j |v_j| / sum_j p_j with
    A = 136 per chunk of a split + 40."""
    scale = 1.0 / math.sqrt(D)
    sdot = np.abs(Kk) @ np.abs(q)                  # [L]
    sc = (Kk @ q) * scale
    p = np.exp(sc - sc.max())
    wabs = (p @ np.abs(Vv)) / p.sum()              # [D]
    A = 136 * chunks_per_split + 40
    return (2 * scale * gamma(D) * sdot.max() + gamma(A) + 2.0 ** -17) * wabs


@pytest.mark.parametrize("shape,ctx,tree,qstd", [
    (FULL, 1024, ("spine", 8), 1.0),
    (FULL, 1024, ("spine", 32), 3.0),
    (FULL, 8192, ("spine", 32), 1.0),
    (FULL, 8192, ("random", 16), 3.0),
    (FULL, 3000, ("random", 29), 1.0),     # ragged: two chunks a split, a short last split
    (FULL, 0, ("bush", 17), 1.0),          # no context: the tree's keys only
    (FULL, 100, ("chain", 1), 3.0),        # one row, one short split
    (FULL, 2500, ("random", 8), 2.0),      # two chunks a split: one load ahead, then an idle slot
    (FULL, 8100, ("spine", 32), 1.0),      # five chunks a split, a ragged last split
    (FULL, 6000, ("bush", 16), 1.0),
    (TINY, 777, ("spine", 32), 1.0),       # heads of 64
    (TINY, 64, ("random", 24), 2.0),
])
def test_attention_identical_inputs(tvs, shape, ctx, tree, qstd):
    kind, n = tree
    parents = {"spine": lambda: synth.spine_tree(n, 11), "random": lambda: synth.random_tree(n, 12),
               "bush": lambda: synth.bush_tree(n), "chain": lambda: synth.chain_tree(n)}[kind]()
    QH, KVH, D = shape.n_qhead, shape.n_kvhead, shape.head_dim
    cap = ctx + n + 5
    _say("attention", shape.name, ctx, kind, n, qstd)
    q = synth.bf16_normal((n, QH * D), 101 + n, qstd)
    K = synth.bf16_normal((KVH, cap, D), 102 + ctx)
    V = synth.bf16_normal((KVH, cap, D), 103 + ctx)
    out = torch.empty((n, QH * D), dtype=torch.bfloat16, device="cuda")
    tvs[shape.name].attention(q.cuda(), K.cuda(), V.cuda(), ctx, parents, out)
    torch.cuda.synchronize()
    gpu = bf16_bits(out.cpu()).reshape(n, QH, D)
    orc = oracle.Oracle(shape, {})
    qf = bf16_bits(q).reshape(n, QH, D)
    Kf, Vf = bf16_bits(K), bf16_bits(V)
    span_chunks = max(1, math.ceil(math.ceil(ctx / 64) / 31))
    exact = np.empty((n, QH, D))
    delta = np.empty((n, QH, D))
    G = QH // KVH
    for t in range(n):
        rows = list(range(ctx)) + [ctx + a for a in _ancestors(parents, t)]
        Kk, Vv = Kf[:, rows], Vf[:, rows]
        exact[t] = orc.attention(qf[t], Kk, Vv)
        for h in range(QH):
            delta[t, h] = _attention_delta(qf[t, h], Kk[h // G], Vv[h // G], D, span_chunks, 33)
    check_rounded(gpu, exact, delta, f"attention {shape.name} ctx={ctx} {kind}{n}")


@pytest.mark.parametrize("ctx", [1024, 3000, 8192])
def test_attention_rows_independent_of_tree_size(tvs, ctx):
    """A node's attention output has the same bits whatever the size of the
    tree around it: the first rows of chains of 4, 8, 24 and 32 nodes (the
    launch gives each block of 32 query rows one wave or, when the CU has
    the waves, two waves that take half of the output dims each) agree
    bit for bit with the same rows of the longest chain."""
    shape = FULL
    QH, KVH, D = shape.n_qhead, shape.n_kvhead, shape.head_dim
    _say("attention rows vs tree size", ctx)
    q = synth.bf16_normal((32, QH * D), 121, 1.0).cuda()
    K = synth.bf16_normal((KVH, ctx + 40, D), 122).cuda()
    V = synth.bf16_normal((KVH, ctx + 40, D), 123).cuda()
    outs = {}
    for n in (32, 24, 8, 4):
        out = torch.empty((n, QH * D), dtype=torch.bfloat16, device="cuda")
        tvs[shape.name].attention(q[:n].contiguous(), K, V, ctx, synth.chain_tree(n), out)
        torch.cuda.synchronize()
        outs[n] = out.cpu()
    for n in (24, 8, 4):
        assert torch.equal(outs[n], outs[32][:n]), f"ctx {ctx}: rows of a {n}-node chain differ"


def test_attention_masks_non_ancestors(tvs):
    """A row does not move when keys and values of nodes off its path change."""
    shape, ctx, n = FULL, 300, 12
    parents = synth.random_tree(n, 5)
    QH, KVH, D = shape.n_qhead, shape.n_kvhead, shape.head_dim
    q = synth.bf16_normal((n, QH * D), 7).cuda()
    K = synth.bf16_normal((KVH, ctx + n, D), 8).cuda()
    V = synth.bf16_normal((KVH, ctx + n, D), 9).cuda()
    a = torch.empty((n, QH * D), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    tvs[shape.name].attention(q, K, V, ctx, parents, a)
    leaf = n - 1
    anc = set(_ancestors(parents, leaf))
    K2, V2 = K.clone(), V.clone()
    for j in range(n):
        if j not in anc:
            K2[:, ctx + j] = -K2[:, ctx + j] * 3
            V2[:, ctx + j] = V2[:, ctx + j] + 7
    tvs[shape.name].attention(q, K2, V2, ctx, parents, b)
    assert torch.equal(a[leaf], b[leaf])
    others = [t for t in range(n) if any(j not in anc for j in _ancestors(parents, t))]
    assert others and not torch.equal(a[others], b[others])


# ------------------------------------------------------------- RoPE + KV

@pytest.mark.parametrize("shape,ctx,n,splits", [
    (FULL, 1024, 32, 9),     # the verify's QKV split count at this width
    (FULL, 8100, 16, 1),     # positions near the end of an 8k table
    (FULL, 0, 1, 4),
    (TINY, 500, 29, 3),
])
def test_rope_kv_identical_inputs(tvs, shape, ctx, n, splits):
    QH, KVH, D = shape.n_qhead, shape.n_kvhead, shape.head_dim
    cols = (QH + 2 * KVH) * D
    _say("rope_kv", shape.name, ctx, n, splits)
    parts = synth.dyadic_partials(splits, n, cols, 200 + n, std=1.5)
    parents = synth.random_tree(n, 201)
    depth = np.array(oracle.node_depths(parents), dtype=np.int32)
    cap = ctx + n + 3
    Kc = torch.zeros((KVH, cap, D), dtype=torch.bfloat16, device="cuda")
    Vc = torch.zeros_like(Kc)
    qo = torch.empty((n, QH * D), dtype=torch.bfloat16, device="cuda")
    tvs[shape.name].rope_kv(torch.from_numpy(synth.splitk_layout(parts)).cuda(), splits, depth, ctx, qo, Kc, Vc)
    torch.cuda.synchronize()
    x = oracle.bf16_round(parts.astype(np.float64).sum(axis=0))   # the projection's rounding point
    orc = oracle.Oracle(shape, {})
    half = D // 2
    gq = bf16_bits(qo.cpu()).reshape(n, QH, D)
    gk = bf16_bits(Kc.cpu())
    gv = bf16_bits(Vc.cpu())
    for t in range(n):
        pos = ctx + int(depth[t])
        q = x[t, :QH * D].reshape(QH, D)
        k = x[t, QH * D:(QH + KVH) * D].reshape(KVH, D)
        v = x[t, (QH + KVH) * D:].reshape(KVH, D)
        # fp32 evaluation of x0 c - x1 s with c, s rounded to fp32: at most
        # four roundings of size 2^-24 |x| each
        for name, src, got in (("q", q, gq[t]), ("k", k, gk[:, ctx + t])):
            mag = np.concatenate([np.abs(src[:, :half]) + np.abs(src[:, half:])] * 2, axis=1)
            check_rounded(got, orc.rope(src, pos), 4 * U * mag + 1e-30, f"rope {name} {shape.name} row {t}")
        assert np.array_equal(gv[:, ctx + t], v), f"v row {t} is not the rounded sum"
    # nothing written outside the tree's slots
    assert not gk[:, :ctx].any() and not gk[:, ctx + n:].any()


# ------------------------------------------------------ residual + RMSNorm

@pytest.mark.parametrize("shape,n,splits", [(FULL, 32, 12), (FULL, 1, 1), (FULL, 8, 3), (TINY, 17, 2)])
def test_resid_norm_identical_inputs(tvs, shape, n, splits):
    H = shape.hidden
    _say("resid_norm", shape.name, n, splits)
    parts = synth.dyadic_partials(splits, n, H, 300 + n, std=0.3)
    x0 = synth.bf16_normal((n, H), 301, 1.0)
    w = synth.bf16_normal((H,), 302, 1.0)
    x = x0.cuda()
    y = torch.empty_like(x)
    tvs[shape.name].resid_norm(torch.from_numpy(synth.splitk_layout(parts)).cuda(), splits, x, w.cuda(), y)
    torch.cuda.synchronize()
    xs = bf16_bits(x0) + oracle.bf16_round(parts.astype(np.float64).sum(axis=0))
    xn = oracle.bf16_round(xs)
    assert np.array_equal(bf16_bits(x.cpu()), xn), "residual stream is not the rounded sum"
    wf = bf16_bits(w)
    exact = np.stack([oracle.rms_norm(xn[t], wf, shape.eps) for t in range(n)])
    # fp32: the sum of squares of H terms (relative gamma_H), then a divide,
    # add, square root and divide (a few ulps), then two multiplies:
    # |y| (gamma_H / 2 + 8u)
    check_rounded(bf16_bits(y.cpu()), exact, np.abs(exact) * (gamma(H) / 2 + 8 * U),
                  f"resid_norm {shape.name} n={n}")


def test_resid_norm_repeated_calls(tvs):
    """Calls in a row on one context with different row counts: each row's
    residual stream and normalised row have the same bits in every call
    (no state carried from one call to the next, a fixed reduction order)."""
    shape = FULL
    H = shape.hidden
    _say("resid_norm repeated", shape.name)
    outs = []
    for n in (32, 5, 32, 17, 32):
        parts = synth.dyadic_partials(4, 32, H, 310, std=0.3)[:, :n]
        x0 = synth.bf16_normal((32, H), 311, 1.0)[:n]
        w = synth.bf16_normal((H,), 312, 1.0)
        x = x0.cuda()
        y = torch.empty_like(x)
        tvs[shape.name].resid_norm(torch.from_numpy(synth.splitk_layout(np.ascontiguousarray(parts))).cuda(), 4,
                                   x, w.cuda(), y)
        torch.cuda.synchronize()
        outs.append((bf16_bits(x.cpu()), bf16_bits(y.cpu())))
    for i, (xb, yb) in enumerate(outs):
        n = xb.shape[0]
        assert np.array_equal(xb, outs[0][0][:n]), f"call {i}: residual stream differs"
        assert np.array_equal(yb, outs[0][1][:n]), f"call {i}: normalised rows differ"


# ------------------------------------------------------- recurrent layer

def _condition_norms(parts, orc):
    """Keep the inputs away from an ambiguous rounding point.  q and k are
    L2-normalised and rounded to bf16 on both sides; the kernel forms the
    normalised value in fp32 (a sum of D squares, a square root, a reciprocal
    and a product: relative error at most gamma_D / 2 + 4u), so an element
    whose exact normalised value lies within that of a bf16 rounding
    midpoint may round either way on a correct implementation, and one such
    element moves the read-out by up to an ulp of q or k times the state.
    Each q or k head-row holding such an element gets its largest
    projection value moved by one bf16 step (in the dyadic partials), which
    rescales the whole normalised row, until none is left.  Returns the
    conditioned partials and the number of rows moved."""
    QH, D = orc.s.n_qhead, orc.s.head_dim
    parts = parts.copy()
    moved = 0
    for _ in range(100):
        x = oracle.bf16_round(parts.astype(np.float64).sum(axis=0))
        n = x.shape[0]
        amb_rows = []
        for blk in (0, 1):
            seg = x[:, blk * QH * D:(blk + 1) * QH * D].reshape(n, QH, D)
            nrm = orc.l2norm(seg)
            dist = np.abs(np.abs(nrm - oracle.bf16_round(nrm)) - oracle.ulp_bf16(nrm) / 2)
            amb = (dist <= (gamma(D) / 2 + 4 * U) * np.abs(nrm)).any(axis=2)
            big = np.argmax(np.abs(seg), axis=2)
            amb_rows += [(t, blk * QH * D + h * D + int(big[t, h])) for t, h in np.argwhere(amb)]
        if not amb_rows:
            return parts, moved
        for t, col in amb_rows:
            parts[0, t, col] += np.float32(max(float(oracle.ulp_bf16(x[t, col])), 2.0 ** -12))
        moved += len(amb_rows)
    raise AssertionError("could not condition the normalised rows")


def _recur_inputs(shape, kind, n, splits, seed, orc):
    QH, D = shape.n_qhead, shape.head_dim
    cols = 3 * QH * D + (2 if kind == synth.DELTA else 1) * QH
    parts, moved = _condition_norms(synth.dyadic_partials(splits, n, cols, seed, std=1.5), orc)
    print(f"[recur inputs] {moved} q/k head-rows moved off a rounding midpoint", flush=True)
    S0 = synth.state0(synth.scaled(shape, "s0", n_layer=1, kinds=[kind]), seed + 1)[0]
    return parts, S0


def _oracle_tree(orc, kind, x, parents, S0):
    """The oracle's sequential read-out of every node from the rounded
    projection rows x [n, cols]: each node steps its parent's state."""
    QH, D = orc.s.n_qhead, orc.s.head_dim
    n = len(parents)
    outs, states = [], []
    for t in range(n):
        prev = S0 if parents[t] < 0 else states[int(parents[t])]
        o, S = orc.recurrent_token(kind, x[t, :3 * QH * D], x[t, 3 * QH * D:], prev, round_out=False)
        outs.append(o)
        states.append(S)
    return np.stack(outs), states


@pytest.mark.parametrize("shape,kind,n,splits,tree", [
    (FULL, synth.RECUR, 16, 4, "spine"),    # the verify's split count for this projection
    (FULL, synth.DELTA, 16, 4, "spine"),
    (FULL, synth.RECUR, 32, 2, "random"),
    (FULL, synth.DELTA, 32, 1, "random"),
    (FULL, synth.DELTA, 1, 3, "chain"),
    (TINY, synth.DELTA, 24, 2, "random"),
    (TINY, synth.RECUR, 9, 1, "bush"),
    # node counts that leave the solver's lanes uneven (nodes t = j, j + 4, ...)
    # and the 16 / 32 coefficient layouts at their edges
    (FULL, synth.DELTA, 5, 4, "random"),
    (FULL, synth.DELTA, 17, 4, "spine"),
    (FULL, synth.DELTA, 31, 4, "random"),
    (TINY, synth.DELTA, 13, 4, "chain"),
])
def test_recur_tree_and_commit_identical_inputs(tvs, shape, kind, n, splits, tree):
    QH, D = shape.n_qhead, shape.head_dim
    parents = {"spine": lambda: synth.spine_tree(n, 21), "random": lambda: synth.random_tree(n, 22),
               "bush": lambda: synth.bush_tree(n), "chain": lambda: synth.chain_tree(n)}[tree]()
    _say("recur_tree", shape.name, "delta" if kind == synth.DELTA else "gated", n, splits, tree)
    orc = oracle.Oracle(synth.scaled(shape, "r", n_layer=1, kinds=[kind]), {})
    parts, S0 = _recur_inputs(shape, kind, n, splits, 400 + n, orc)
    tv = tvs[shape.name]
    out = torch.empty((n, QH * D), dtype=torch.bfloat16, device="cuda")
    sk = torch.zeros((32, QH, D), dtype=torch.bfloat16, device="cuda")
    sv = torch.zeros((32, QH, D), dtype=torch.float32, device="cuda")
    sg = torch.zeros((32, QH), dtype=torch.float32, device="cuda")
    state = S0.cuda()
    tv.recur_tree(kind, torch.from_numpy(synth.splitk_layout(parts)).cuda(), splits, parents, state, out,
                  sk, sv, sg)
    torch.cuda.synchronize()
    x = oracle.bf16_round(parts.astype(np.float64).sum(axis=0))
    S0f = S0.double().numpy()
    exact, states = _oracle_tree(orc, kind, x, parents, S0f)
    exact = exact.reshape(n, QH, D)
    # delta per (node, head, value column): the read-out is
    # e^{gc_t} S0^T q_t + sum over ancestors-or-self s of e^{gc_t - gc_s} (q_t . k_s) u_s.
    # S0 enters the matrix cores as bf16 high + low parts (relative 2^-17)
    # over 2 D products (gamma_2D); the coefficients carry gamma_D |q||k| and
    # exp's ulps; the sum over at most 32 nodes gamma_32.  The oracle's own
    # state is rounded to fp32 after each of its depth+1 steps.  T1 and T2
    # below are the magnitudes of the two terms, u_s recovered from the
    # oracle's consecutive states (S_s - e^{g_s} S_parent = k_s u_s^T).
    qn = np.stack([orc.r(orc.l2norm(x[t, :QH * D].reshape(QH, D))) for t in range(n)])
    kn = np.stack([orc.r(orc.l2norm(x[t, QH * D:2 * QH * D].reshape(QH, D))) for t in range(n)])
    g = oracle.log_sigmoid(x[:, 3 * QH * D:3 * QH * D + QH])      # [n, QH]
    depth = oracle.node_depths(parents)
    gc = np.zeros((n, QH))
    u = np.zeros((n, QH, D))
    for t in range(n):
        p = int(parents[t])
        gc[t] = g[t] + (gc[p] if p >= 0 else 0.0)
        prev = S0f if p < 0 else states[p]
        dS = states[t] - np.exp(g[t])[:, None, None] * prev
        u[t] = np.einsum("hk,hkv->hv", kn[t], dS) / np.sum(kn[t] * kn[t], axis=1, keepdims=True)
    delta = np.empty((n, QH, D))
    for t in range(n):
        anc = _ancestors(parents, t)
        T1 = np.exp(gc[t])[:, None] * np.einsum("hk,hkv->hv", np.abs(qn[t]), np.abs(S0f))
        T2 = np.zeros((QH, D))
        for s in anc:
            coef = np.exp(gc[t] - gc[s]) * np.abs(np.sum(qn[t] * kn[s], axis=1))
            T2 += coef[:, None] * np.abs(u[s])
        Sabs = np.einsum("hk,hkv->hv", np.abs(qn[t]), np.abs(states[t]))
        delta[t] = ((2.0 ** -17 + gamma(2 * D)) * T1 + (gamma(D) + gamma(32) + 8 * U) * (T1 + T2)
                    + (depth[t] + 1) * U * Sabs)
    gpu = bf16_bits(out.cpu()).reshape(n, QH, D)
    name = f"recur_tree {shape.name} {'delta' if kind == synth.DELTA else 'gated'} n={n}"
    check_rounded(gpu, exact, delta, name)
    # the saved keys are the normalised bf16 keys of every node
    assert np.array_equal(bf16_bits(sk.cpu())[:n], kn), f"{name}: saved keys"
    np.testing.assert_allclose(sg.cpu().numpy()[:n], gc, rtol=0, atol=1e-5 * (1 + np.abs(gc).max()))

    # commit the deepest path (the longest root-to-node path) and compare the
    # state with the oracle's state after its last node
    leaf = int(np.argmax(depth))
    path = _ancestors(parents, leaf)
    tv.recur_commit(state, sk, sv, sg, path)
    torch.cuda.synchronize()
    got = state.cpu().double().numpy()
    want = states[leaf]
    # e^{gc_L} S0 + sum over the path of e^{gc_L - gc_t} k_t u_t^T in fp32
    # (L + 2 roundings per element) against the oracle's L fp32 roundings.
    # A delta layer's pseudo-values come from the kernel's forward
    # substitution; each carries the read-out's kind of error, bounded by
    # du_t = b_t e^{gc_t}(2^-17 + gamma_2D) |S0|^T |k_t| + (gamma_D + gamma_32 + 8u)
    # (|b_t v_t| + b_t e^{gc_t} |S0|^T |k_t| + sum over strict ancestors s of
    # b_t e^{gc_t - gc_s} |k_t . k_s| |u_s|), which enters the state through k_t.
    mag = np.exp(gc[leaf])[:, None, None] * np.abs(S0f)
    du = np.zeros((n, QH, D))
    if kind == synth.DELTA:
        b = oracle.sigmoid(x[:, 3 * QH * D + QH:3 * QH * D + 2 * QH])      # [n, QH]
        v = x[:, 2 * QH * D:3 * QH * D].reshape(n, QH, D)
        for t in range(n):
            s0k = np.exp(gc[t])[:, None] * np.einsum("hk,hkv->hv", np.abs(kn[t]), np.abs(S0f))
            acc = np.abs(v[t]) + s0k
            for s in _ancestors(parents, t)[:-1]:
                acc = acc + (np.exp(gc[t] - gc[s]) * np.abs(np.sum(kn[t] * kn[s], axis=1)))[:, None] * np.abs(u[s])
            du[t] = b[t][:, None] * ((2.0 ** -17 + gamma(2 * D)) * s0k + (gamma(D) + gamma(32) + 8 * U) * acc)
    extra = np.zeros_like(mag)
    for t in path:
        w = np.exp(gc[leaf] - gc[t])[:, None, None] * np.abs(kn[t])[:, :, None]
        mag = mag + w * np.abs(u[t])[:, None, :]
        extra = extra + w * du[t][:, None, :]
    L = len(path)
    tol = (2 * L + 8) * U * mag + extra
    err = np.abs(got - want)
    print(f"[{name} commit] path {len(path)}, max err {err.max():.3g}, max tol {tol.max():.3g}", flush=True)
    assert (err <= tol + 1e-30).all(), f"{name}: committed state off by {err.max():.3g}"


# ------------------------------------------------------------- KV gather

@pytest.mark.parametrize("ctx,n", [(1024, 32), (0, 5), (8190 - 32, 32)])
def test_gather_kv_is_a_plain_gather(tvs, ctx, n):
    shape = FULL
    KVH, D = shape.n_kvhead, shape.head_dim
    cap = ctx + n + 2
    K = synth.bf16_normal((KVH, cap, D), 500 + ctx).cuda()
    V = synth.bf16_normal((KVH, cap, D), 501 + ctx).cuda()
    parents = synth.random_tree(n, 502)
    path = _ancestors(parents, n - 1)
    K0, V0 = K.cpu(), V.cpu()
    tvs[shape.name].gather_kv(K, V, ctx, path)
    torch.cuda.synchronize()
    K1, V1 = K.cpu(), V.cpu()
    for d, node in enumerate(path):
        assert torch.equal(K1[:, ctx + d], K0[:, ctx + node]) and torch.equal(V1[:, ctx + d], V0[:, ctx + node])
    keep = [i for i in range(cap) if not (ctx <= i < ctx + len(path))]
    assert torch.equal(K1[:, keep], K0[:, keep]) and torch.equal(V1[:, keep], V0[:, keep])


def test_kernel_calls_reject_bad_arguments(tvs):
    from greedy_draft_tree_amd import TVError
    tv = tvs[FULL.name]
    shape = FULL
    QH, KVH, D = shape.n_qhead, shape.n_kvhead, shape.head_dim
    q = torch.zeros((4, QH * D), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((KVH, 10, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(TVError):          # ctx + rows beyond the cache
        tv.attention(q, K, K, 8, [-1, 0, 1, 2], out)
    with pytest.raises(TVError):          # not a tree
        tv.attention(q, K, K, 0, [-1, 2, 0, 1], out)
    with pytest.raises(TVError):          # a path that moves a row down
        tv.gather_kv(K, K, 0, [0, 2, 1])
