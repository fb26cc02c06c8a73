"""Pins of the oracle's numeric primitives against the pages and libraries."""
import os

import numpy as np
import pytest
import torch

import oracle
from synth import Modifiers

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(path):
    out = []
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


def test_ulp_bf16_page_example():
    # "Exactness", Parallel requests: one BF16 step at magnitude 16..32 is 0.125.
    for v, u in _rows(os.path.join(GOLD, "ulp_bf16.txt")):
        assert float(oracle.ulp_bf16(float(v))) == float(u), v


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39])      # subnormal range
    x32 = x.astype(np.float32)
    # exact ties between two bf16 neighbours, both parities
    base = torch.randn(2000).to(torch.bfloat16).to(torch.float32).numpy()
    ties = base + np.float32(0.5) * oracle.ulp_bf16(base).astype(np.float32)
    x32 = np.concatenate([x32, ties.astype(np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x32.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_ulp_is_bf16_spacing():
    # ulp(x) is the distance to the next bf16 value above |x| (normal range).
    vals = torch.randn(5000).to(torch.bfloat16)
    bits = vals.view(torch.int16).numpy().astype(np.int32) & 0x7FFF
    up = torch.from_numpy((bits + 1).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    here = np.abs(vals.to(torch.float64).numpy())
    np.testing.assert_array_equal(up - here, oracle.ulp_bf16(here))


@pytest.mark.parametrize("N,K", [(1, 1), (7, 33), (130, 517), (64, 4096)])
def test_matvec_matches_numpy(N, K):
    g = torch.Generator().manual_seed(N * 1000 + K)
    W = (torch.randn(N, K, generator=g) * 0.5).to(torch.bfloat16)
    x = torch.randn(K, generator=g, dtype=torch.float64).numpy()
    m = oracle.Oracle.__new__(oracle.Oracle)
    m.W = {"w": oracle.t2u16(W)}
    m.lib = oracle._load()
    got = m.matvec("w", x)
    want = W.to(torch.float64).numpy() @ x
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_matvec_thread_count_invariant():
    g = torch.Generator().manual_seed(5)
    W = torch.randn(300, 1000, generator=g).to(torch.bfloat16)
    x = torch.randn(1000, generator=g, dtype=torch.float64).numpy()
    m = oracle.Oracle.__new__(oracle.Oracle)
    m.W = {"w": oracle.t2u16(W)}
    m.lib = oracle._load()
    t0 = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = m.matvec("w", x)
        oracle.set_threads(7)
        b = m.matvec("w", x)
    finally:
        oracle.set_threads(t0)
    np.testing.assert_array_equal(a, b)


def test_modifiers_worked_example():
    rows = _rows(os.path.join(GOLD, "modifiers_example.txt"))
    logits = np.array([float(v) for v in rows[0]])
    prior = [int(v) for v in rows[1]]
    theta = float(rows[2][0])
    bias = [(int(a), float(b)) for a, b in rows[3:5]]
    allowed = [int(v) for v in rows[5]]
    want = np.array([float(v) for v in rows[6]])
    am, l1, l2 = int(rows[7][0]), float(rows[7][1]), float(rows[7][2])
    V = len(logits)
    words = np.zeros(1, dtype=np.uint32)
    for a in allowed:
        words[0] |= np.uint32(1 << a)
    mods = Modifiers(theta, np.array([b[0] for b in bias], np.int32),
                     np.array([b[1] for b in bias], np.float32), words)
    s = oracle.apply_modifiers(logits, prior, mods)
    np.testing.assert_array_equal(s.astype(np.float64), want)
    a, t1, t2, gap = oracle.top2(s)
    assert (a, t1, t2) == (am, l1, l2)
    assert gap == (l1 - l2) / oracle.ulp_bf16(l1)


def test_top2_tie_goes_to_lowest_id():
    s = np.array([0.5, 2.0, -1.0, 2.0, 1.9], dtype=np.float32)
    a, l1, l2, gap = oracle.top2(s)
    assert a == 1 and l1 == 2.0 and l2 == 2.0 and gap == 0.0


def test_top2_all_masked_but_one():
    s = np.full(10, -np.inf, dtype=np.float32)
    s[7] = -3.0
    a, l1, l2, gap = oracle.top2(s)
    assert a == 7 and gap == np.inf


def test_top2_matches_sort():
    rng = np.random.default_rng(3)
    for _ in range(50):
        s = rng.standard_normal(1000).astype(np.float32) * 3
        order = np.argsort(-s.astype(np.float64), kind="stable")
        a, l1, l2, _ = oracle.top2(s)
        assert a == order[0] and l1 == s[order[0]] and l2 == s[order[1]]


def test_penalty_uses_ieee_fp32_division():
    # l / 1.1 is taken in fp32 (the precision of the logits), not fp64.
    x = np.float32(3.3)
    mods = Modifiers(1.1, np.zeros(0, np.int32), np.zeros(0, np.float32), None)
    s = oracle.apply_modifiers(np.array([x], dtype=np.float64), [0], mods)
    assert s[0] == np.float32(x) / np.float32(1.1)
