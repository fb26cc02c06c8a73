"""The oracle's recurrent-layer wiring against a one-head example worked by
hand (tests/golden/recurrent_wiring.txt).

The wiring pinned here: which wqkv rows are q, k and v; the L2 norms of q
and k; the gate g = log sigmoid(x W_a) and the delta layer's write strength
b = sigmoid(x W_b) from the rows stacked under the gate rows; the state
update and the read-out o = S^T q with the key index first.  Swapping any
two of q, k and v, dropping a norm, using sigmoid in place of log sigmoid,
transposing the state or the read-out all change these numbers.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "recurrent_wiring.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, *v = line.split()
            out[k] = np.array([float(x) for x in v])
    return out


def _oracle(kind):
    shape = synth.ModelShape("wiring", 1, 2, 1, 1, 2, 8, 4, (kind,))
    bf = lambda rows: torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    wqkv = bf([[3, 0], [0, 4], [0, 0], [1, 1], [2, -1], [-1, -1]])
    wa = bf([[0.5, 0.5]] if kind == synth.RECUR else [[0.5, 0.5], [-0.25, -0.75]])
    return oracle.Oracle(shape, {"layers.0.wqkv": wqkv, "layers.0.wa": wa}, exact=True)


@pytest.mark.parametrize("kind,name", [(synth.RECUR, "gated"), (synth.DELTA, "delta")])
def test_recurrent_layer_matches_hand_worked_example(kind, name):
    g = _golden()
    orc = _oracle(kind)
    S0 = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    o, S = orc.recurrent_layer(0, np.array([1.0, 1.0]), S0)
    np.testing.assert_allclose(S.reshape(-1), g[f"{name}_S"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(o, g[f"{name}_o"], rtol=1e-6, atol=0)


def test_example_tells_the_layer_kinds_apart():
    g = _golden()
    assert np.abs(g["gated_o"] - g["delta_o"]).min() > 0.1
    assert abs(g["sigma1"] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15
