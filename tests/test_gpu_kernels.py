"""Per-kernel parity of the skinny GEMM and the fp32 head (MI355X only).

Inputs are seeded synthetic bf16 operands from ``synth``'s generator; the
expected values are the oracle's fp64 dot products.

* fp32 outputs: |y - y64| <= gamma_K * sum_k |x_k w_k| (Higham's bound for a
  length-K fp32 sum, gamma_K = K u / (1 - K u), u = 2^-24), and the north
  star's 1e-5 relative bound for the head accumulation.
* bf16 outputs: equal to the fp64 value rounded to bf16, except where the
  fp64 value lies within the fp32 error bound of a rounding boundary.
* Row invariance ("Exactness", The one exception: near ties, and Parallel
  requests): a row's result is bit-identical for every row count 1..32 and
  every row slot.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def tv():
    _gpu()
    from greedy_draft_tree_amd import TreeVerifier
    s = torch.cuda.current_stream().cuda_stream
    t = TreeVerifier.for_shape(synth.C1, max_ctx=64, max_req=1, stream=s)
    return t


def _ref(x_bf16, w_bf16):
    """fp64 products and the sum of |terms| per output, via the oracle's
    plain matvec."""
    m = oracle.Oracle.__new__(oracle.Oracle)
    m.lib = oracle._load()
    m.W = {"w": oracle.t2u16(w_bf16.cpu())}
    wa = w_bf16.cpu().to(torch.float64).abs()
    m.W["wa"] = oracle.t2u16(wa.to(torch.bfloat16))  # |w| is exact in bf16
    x = x_bf16.cpu().to(torch.float64).numpy()
    y = np.stack([m.matvec("w", x[i]) for i in range(x.shape[0])])
    a = np.stack([m.matvec("wa", np.abs(x[i])) for i in range(x.shape[0])])
    return y, a


def _operands(M, N, K, seed, xstd=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = (torch.randn(M, K, generator=g, device="cuda") * xstd).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    return x, w


def _packed_layout(w):
    """The packed order documented in include/treeverify.h, built on the host
    from a row-major matrix (tiles of 32 rows, steps of 64 k, pieces (q, hf)
    of 8 k values in order 2q+hf, present pieces only)."""
    N, K = w.shape
    src = w.cpu().view(torch.int16).numpy()
    out = np.empty(N * K, dtype=np.int16)
    pos = 0
    for t in range(0, N, 32):
        nr = min(32, N - t)
        for s in range(0, K, 64):
            kr = min(64, K - s)
            for pi in range(8):
                q, hf = pi >> 1, pi & 1
                k0 = 32 * hf + 8 * q
                if k0 >= kr:
                    continue
                for c in range(nr):
                    out[pos:pos + 8] = src[t + c, s + k0:s + k0 + 8]
                    pos += 8
    assert pos == N * K
    return out


@pytest.mark.parametrize("N,K", [(64, 128), (40, 200), (100, 688)])
def test_pack_weight_matches_documented_layout(tv, N, K):
    _, w = _operands(1, N, K, N + K)
    want = _packed_layout(w)
    tv.pack_weight(w)
    got = w.cpu().view(torch.int16).numpy().reshape(-1)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (7, 1000, 688), (32, 7168, 5120), (13, 5120, 17408),
                                   (32, 33, 5128), (5, 40, 5120), (32, 17408, 5120), (8, 5120, 5120)])
def test_linear_fp32_within_higham_bound(tv, M, N, K):
    x, w = _operands(M, N, K, M * 7 + N)
    ref, absum = _ref(x, w)
    tv.pack_weight(w)
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tv.linear(x, w, y)
    gam = K * U / (1 - K * U)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert (err <= gam * absum + 1e-30).all(), float((err / (gam * absum + 1e-30)).max())


@pytest.mark.parametrize("M,N,K", [(3, 512, 256), (32, 7168, 5120), (9, 17408, 5120)])
def test_linear_bf16_is_correctly_rounded(tv, M, N, K):
    x, w = _operands(M, N, K, 100 + M)
    ref, absum = _ref(x, w)
    tv.pack_weight(w)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tv.linear(x, w, y)
    want = oracle.bf16_round(ref)
    got = y.cpu().to(torch.float64).numpy()
    gam = K * U / (1 - K * U)
    # where rounding differs, the fp64 value must sit within the fp32 bound of
    # the midpoint between the two bf16 neighbours
    bad = got != want
    mid = (got + want) / 2
    near = np.abs(ref - mid) <= gam * absum + 2 * U * np.abs(ref)
    assert (~bad | near).all(), int((bad & ~near).sum())
    assert bad.mean() < 1e-3


def test_linear_rows_bitwise_invariant(tv):
    N, K = 4096, 5120
    x, w = _operands(32, N, K, 5)
    tv.pack_weight(w)
    full = torch.empty(32, N, dtype=torch.float32, device="cuda")
    tv.linear(x, w, full)
    full_b = torch.empty(32, N, dtype=torch.bfloat16, device="cuda")
    tv.linear(x, w, full_b)
    rng = np.random.default_rng(0)
    for M in (1, 2, 5, 8, 16, 17, 24, 31, 32):
        perm = rng.permutation(32)[:M]
        xs = x[torch.from_numpy(perm).cuda()].contiguous()
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        tv.linear(xs, w, y)
        assert torch.equal(y, full[torch.from_numpy(perm).cuda()]), M
        yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tv.linear(xs, w, yb)
        assert torch.equal(yb, full_b[torch.from_numpy(perm).cuda()]), M


@pytest.fixture(scope="module")
def head(tv):
    w = synth.weights(synth.C1, seed=0, device="cuda", only=["head"])["head"]
    host = w.cpu()
    tv.bind("head", w)
    return host


def test_head_top2_c1(tv, head):
    M = 32
    g = torch.Generator(device="cuda").manual_seed(11)
    x = torch.randn(M, synth.C1.hidden, generator=g, device="cuda").to(torch.bfloat16)
    logits = torch.empty(M, synth.C1.vocab, dtype=torch.float32, device="cuda")
    am, gap = tv.head_top2(x, logits)
    gl = logits.cpu().numpy().astype(np.float64)
    ref, absum = _ref(x, head)
    K = synth.C1.hidden
    gam = K * U / (1 - K * U)
    err = np.abs(gl - ref)
    assert (err <= gam * absum).all()
    # spec head bound: 1e-5 relative (to the row's largest |logit|)
    assert (err.max(axis=1) <= 1e-5 * np.abs(ref).max(axis=1)).all()
    for i in range(M):
        a, l1, l2, g2 = oracle.top2(gl[i])
        assert am[i] == a and gap[i] == np.float32(g2)
        a64, _, _, g64 = oracle.top2(oracle.f32(ref[i]))
        assert am[i] == a64 or g64 <= 1.0


def test_head_rows_bitwise_invariant(tv, head):
    g = torch.Generator(device="cuda").manual_seed(12)
    x = torch.randn(32, synth.C1.hidden, generator=g, device="cuda").to(torch.bfloat16)
    full = torch.empty(32, synth.C1.vocab, dtype=torch.float32, device="cuda")
    am_full, gap_full = tv.head_top2(x, full)
    for M, rows in ((1, [31]), (8, list(range(8, 16))), (3, [30, 0, 17])):
        xs = x[rows].contiguous()
        out = torch.empty(M, synth.C1.vocab, dtype=torch.float32, device="cuda")
        am, gap = tv.head_top2(xs, out)
        assert torch.equal(out, full[rows])
        np.testing.assert_array_equal(am, am_full[rows])
        np.testing.assert_array_equal(gap, gap_full[rows])


# ------------------------------------------------------------ dense (prefill) GEMM

@pytest.mark.parametrize("M,N,K", [(33, 512, 256), (130, 1056, 1024), (300, 5120, 5120), (97, 17408, 512),
                                   (1000, 17408, 512),    # 256 x 256 tiles, a ragged last row tile
                                   (500, 5120, 1280)])    # 64-row tiles, a ragged last row tile
def test_dense_linear_fp32_and_bf16(tv, M, N, K):
    """More than 32 rows run the dense kernel: fp32 sums within Higham's
    bound, bf16 outputs correctly rounded up to that bound."""
    x, w = _operands(M, N, K, 300 + M)
    ref, absum = _ref(x, w)
    tv.pack_weight(w)
    gam = K * U / (1 - K * U)
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tv.linear(x, w, y)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
    assert (err <= gam * absum + 1e-30).all(), float((err / (gam * absum + 1e-30)).max())
    yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tv.linear(x, w, yb)
    want = oracle.bf16_round(ref)
    got = yb.cpu().to(torch.float64).numpy()
    bad = got != want
    mid = (got + want) / 2
    near = np.abs(ref - mid) <= gam * absum + 2 * U * np.abs(ref)
    assert (~bad | near).all(), int((bad & ~near).sum())
    # the bf16 output is the fp32 sum rounded once
    assert torch.equal(yb, y.to(torch.bfloat16))


@pytest.mark.parametrize("N,K,R", [(2048, 1024, 300), (17408, 512, 512), (17408, 1280, 1024), (7168, 1280, 2048),
                                   (7168, 1280, 1024), (5120, 1280, 768), (5120, 1280, 512)])
def test_dense_linear_rows_bitwise_invariant(tv, N, K, R):
    """A row's dense result does not depend on the row count, its slot, or
    the tile shape the row count selects (at 17408 columns 512 rows take 4
    row groups per workgroup, fewer rows take 2; 1024 rows take the 256 x
    256 tiles with the last weight blocks on 64-row tiles; 128-row tiles at
    7168 columns for 1024 and 2048 rows, 64-row tiles at 5120 columns for 512
    and 768 rows; the subsets below on the 32-row-group kernel)."""
    x, w = _operands(R, N, K, 7)
    tv.pack_weight(w)
    full = torch.empty(R, N, dtype=torch.float32, device="cuda")
    tv.linear(x, w, full)
    rng = np.random.default_rng(1)
    for M in (33, 64, 127, 129, 257):
        perm = torch.from_numpy(rng.permutation(R)[:M]).cuda()
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        tv.linear(x[perm].contiguous(), w, y)
        assert torch.equal(y, full[perm]), M


def test_head_top2_exact_ties_go_to_the_lowest_id():
    """Planted exact ties: head rows 5, 700 and 1000 are identical, so their
    fp32 logits are bitwise equal; they are the largest of the row, so the
    top-2 reduce must return the lowest of them with a gap of 0, and a
    second planted pair (rows 2 and 3, the only rows above the rest in row
    1's input) the same.  Ties are decided under a strict order, so this
    holds for any merge order of the candidates."""
    _gpu()
    from greedy_draft_tree_amd import TreeVerifier
    shape = synth.C0
    s = torch.cuda.current_stream().cuda_stream
    t = TreeVerifier.for_shape(shape, max_ctx=64, max_req=1, stream=s)
    H, V = shape.hidden, shape.vocab
    g = torch.Generator(device="cpu").manual_seed(3)
    w = (torch.randn(V, H, generator=g) * 0.02).to(torch.bfloat16)
    w[5] = w[700] = w[1000] = 0.05
    w[2] = w[3] = torch.linspace(-0.06, 0.06, H).to(torch.bfloat16)
    t.bind("head", w.cuda())
    x = torch.ones(2, H, dtype=torch.bfloat16)
    x[1] = torch.linspace(-1, 1, H).to(torch.bfloat16)
    logits = torch.empty(2, V, dtype=torch.float32, device="cuda")
    am, gap = t.head_top2(x.cuda(), logits)
    lg = logits.cpu()
    assert lg[0, 5] == lg[0, 700] == lg[0, 1000] and int(lg[0].argmax()) in (5, 700, 1000)
    assert am[0] == 5 and gap[0] == 0.0
    assert lg[1, 2] == lg[1, 3] and float(lg[1, 2]) > float(lg[1, 4:].max())
    assert am[1] == 2 and gap[1] == 0.0
    t.close()
