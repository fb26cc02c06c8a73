"""Tree-verify pass of greedy speculative decoding on MI355X (gfx950).

A thin ctypes binding over ``libtreeverify.so`` (C ABI in
``include/treeverify.h``).  It only marshals arguments: every step of the
pass runs in the library's HIP kernels.  PyTorch supplies device memory and
the stream.  Importing this package fails loudly if the library is missing.
"""
from .binding import (TV_EHIP, TV_ECAPACITY, TV_EINVAL, TV_ESTATE, TV_LAYER_ATTN,
                      TV_LAYER_DELTA, TV_LAYER_RECUR, TV_MAX_NODES, TV_OK, TreeVerifier, TVError,
                      accept_walk, exported_symbols, library_path, load_library)

__all__ = ["TreeVerifier", "TVError", "accept_walk", "load_library", "library_path",
           "exported_symbols", "TV_OK", "TV_EINVAL", "TV_ECAPACITY", "TV_ESTATE", "TV_EHIP",
           "TV_MAX_NODES", "TV_LAYER_ATTN", "TV_LAYER_RECUR", "TV_LAYER_DELTA"]
