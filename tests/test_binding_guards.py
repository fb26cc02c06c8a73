"""The binding rejects unusable tensors before any library call (CPU only).

The library writes through raw device pointers, so a logits tensor of the
wrong element size, on the host, non-contiguous or too small would be
written past its end on the GPU.  Every entry point that takes a tensor
checks dtype, layout, device and size first; here the library handle is a
stub that fails the test if it is ever reached.
"""
import numpy as np
import pytest
import torch

from greedy_draft_tree_amd import binding
from greedy_draft_tree_amd.binding import TreeVerifier, check_device_tensor


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"library function {name} was called")


def _verifier(vocab=64, hidden=32):
    tv = TreeVerifier.__new__(TreeVerifier)
    tv.lib = _NoCalls()
    tv.h = None
    tv.vocab, tv.hidden, tv.max_ctx, tv.max_req = vocab, hidden, 128, 1
    tv._keep = {}
    return tv


class _FakeCuda:
    """Stands in for a device tensor: passes the device check, so the other
    checks are exercised on their own."""

    def __init__(self, t):
        self.t = t
        self.is_cuda = True
        self.dtype = t.dtype
        self.shape = t.shape

    def is_contiguous(self):
        return self.t.is_contiguous()

    def numel(self):
        return self.t.numel()

    def dim(self):
        return self.t.dim()


PARENTS = [-1, 0, 1]
TOKENS = [1, 2, 3]


@pytest.mark.parametrize("bad", [
    _FakeCuda(torch.zeros(3, 64, dtype=torch.bfloat16)),      # 2-byte elements: the head writes 4
    _FakeCuda(torch.zeros(3, 64, dtype=torch.float16)),
    _FakeCuda(torch.zeros(2, 64, dtype=torch.float32)),       # too small for 3 rows
    _FakeCuda(torch.zeros(64, 3, dtype=torch.float32).t()),   # not contiguous
    torch.zeros(3, 64, dtype=torch.float32),                  # on the host
])
def test_logits_guard_every_entry_point(bad):
    tv = _verifier()
    with pytest.raises(ValueError):
        tv.verify_tree(0, PARENTS, TOKENS, logits=bad)
    with pytest.raises(ValueError):
        tv.round(0, PARENTS, TOKENS, logits=bad)
    with pytest.raises(ValueError):
        tv.verify_trees([0], [PARENTS], [TOKENS], logits=bad)
    with pytest.raises(ValueError):
        tv.residual_round(0, PARENTS, TOKENS, 1.0, [0.5] * 3, logits=bad)


def test_head_top2_checks_x_and_logits():
    tv = _verifier()
    good_logits = _FakeCuda(torch.zeros(2, 64, dtype=torch.float32))
    for bad_x in (_FakeCuda(torch.zeros(2, 32, dtype=torch.float32)),   # not bf16
                  _FakeCuda(torch.zeros(2, 16, dtype=torch.bfloat16)),  # wrong width
                  _FakeCuda(torch.zeros(33, 32, dtype=torch.bfloat16)), # too many rows
                  torch.zeros(2, 32, dtype=torch.bfloat16)):            # host
        with pytest.raises(ValueError):
            tv.head_top2(bad_x, good_logits)
    x = _FakeCuda(torch.zeros(2, 32, dtype=torch.bfloat16))
    for bad_l in (_FakeCuda(torch.zeros(2, 64, dtype=torch.bfloat16)),
                  _FakeCuda(torch.zeros(1, 64, dtype=torch.float32))):
        with pytest.raises(ValueError):
            tv.head_top2(x, bad_l)


def test_linear_and_pack_check_operands():
    tv = _verifier()
    x = _FakeCuda(torch.zeros(4, 64, dtype=torch.bfloat16))
    w = _FakeCuda(torch.zeros(8, 64, dtype=torch.bfloat16))
    y = _FakeCuda(torch.zeros(4, 8, dtype=torch.float32))
    with pytest.raises(ValueError):   # x not bf16
        tv.linear(_FakeCuda(torch.zeros(4, 64, dtype=torch.float32)), w, y)
    with pytest.raises(ValueError):   # w of another K
        tv.linear(x, _FakeCuda(torch.zeros(8, 32, dtype=torch.bfloat16)), y)
    with pytest.raises(ValueError):   # y of another shape
        tv.linear(x, w, _FakeCuda(torch.zeros(4, 9, dtype=torch.float32)))
    with pytest.raises(ValueError):   # y of an unsupported dtype
        tv.linear(x, w, _FakeCuda(torch.zeros(4, 8, dtype=torch.float16)))
    with pytest.raises(ValueError):   # host operand
        tv.linear(torch.zeros(4, 64, dtype=torch.bfloat16), w, y)
    with pytest.raises(ValueError):
        tv.pack_weight(_FakeCuda(torch.zeros(8, 64, dtype=torch.float32)))


def test_bind_rejects_host_tensor():
    tv = _verifier()
    with pytest.raises(ValueError):
        tv.bind("emb", torch.zeros(4, 4, dtype=torch.bfloat16))


def test_check_device_tensor_accepts_a_good_tensor():
    check_device_tensor(_FakeCuda(torch.zeros(3, 64, dtype=torch.float32)), "x", "float32", 3 * 64)
    assert binding._logits_ptr(None, 3, 64, "x") is None
