"""The bench's algorithmic byte count per verify against the per-verify
totals tabulated in the hot-path scope (weights once + KV read + tree KV
written + fp32 logits, with a one-token commit), to the printed precision."""
import pytest

import bench
import synth


@pytest.mark.parametrize("shape,n,ctxs,gb", [
    (synth.C1, 8, [1024], 2.2256), (synth.C1, 16, [1024], 2.2306), (synth.C1, 24, [1024], 2.2356),
    (synth.C1, 32, [1024], 2.2405),
    (synth.C2, 8, [1024], 44.110), (synth.C2, 16, [1024], 44.117), (synth.C2, 24, [1024], 44.124),
    (synth.C2, 32, [1024], 44.131),
    (synth.C2, 8, [8192], 45.989), (synth.C2, 32, [8192], 46.010),
])
def test_verify_bytes_match_table(shape, n, ctxs, gb):
    b = bench.model_bytes(shape, n, ctxs, [1] * len(ctxs)) / 1e9
    # the table leaves out the committed row move (2 x 2 x 1 row x KVH x D x 2 bytes per layer)
    commit = len(shape.kinds) * 2 * 2 * shape.n_kvhead * shape.head_dim * 2 / 1e9
    digits = 4 if gb < 10 else 3
    assert round(b - commit, digits) == pytest.approx(gb, abs=1.5 * 10 ** -digits), (b, gb)


def test_two_request_bytes():
    # two requests of 16 rows at contexts 1024 and 8192 with modifiers: 46.28 GB on the 64-layer stack
    b = bench.model_bytes(synth.C2, 16, [1024, 8192], [1, 1], mods=True) / 1e9
    assert b == pytest.approx(46.28, abs=0.01)
