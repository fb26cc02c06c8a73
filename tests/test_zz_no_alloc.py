"""tv_linear_noalloc against tv_linear (MI355X only).

The allocation-free variant runs the same projection kernels on a static
per-GPU scratch array; its outputs must equal tv_linear's bit for bit.  Two
calls in a row share the array, the second smaller than the first, and each
is checked; a shape whose scratch does not fit is refused before any work.
"""
import ctypes

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _operands(M, N, K, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    return x, w


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_linear_on_two_calls(dtype):
    _gpu()
    from greedy_draft_tree_amd import TreeVerifier, binding
    stream = torch.cuda.current_stream().cuda_stream
    tv = TreeVerifier.for_shape(synth.C1, max_ctx=64, max_req=1, stream=stream)
    try:
        # a split-K shape (QKV at full width, 32 rows), then a smaller one,
        # then a many-row (dense kernel) one
        for M, N, K, seed in ((32, 7168, 5120, 1), (5, 1000, 688, 2), (70, 640, 512, 3)):
            print(f"[case] no-alloc linear M={M} N={N} K={K} {dtype}", flush=True)
            x, w = _operands(M, N, K, seed)
            tv.pack_weight(w)
            want = torch.empty(M, N, dtype=dtype, device="cuda")
            tv.linear(x, w, want)
            got = torch.full((M, N), float("nan"), dtype=dtype, device="cuda")
            binding.linear_noalloc(x, w, got, stream)
            torch.cuda.synchronize()
            assert torch.equal(got, want), (M, N, K)
    finally:
        tv.close()


def test_noalloc_refuses_oversized_scratch():
    _gpu()
    from greedy_draft_tree_amd import TV_EINVAL, binding
    lib = binding.load_library()
    buf = torch.zeros(16, dtype=torch.float32, device="cuda")
    # fp32 output at 32 rows and 2^20 columns needs 32 * 8192 * 16 B = 4 MiB + 
    # of candidates: refused before any launch (the buffers are never touched)
    rc = lib.tv_linear_noalloc(buf.data_ptr(), buf.data_ptr(), 32, (1 << 20) + 128, 64, buf.data_ptr(), 1,
                               ctypes.c_void_p(0))
    assert rc == TV_EINVAL
    assert b"static scratch" in lib.tv_last_error(None)
    torch.cuda.synchronize()
    assert not buf.any()
