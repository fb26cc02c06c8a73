"""ctypes binding of the C ABI (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

TV_OK, TV_EINVAL, TV_ECAPACITY, TV_ESTATE, TV_EHIP = 0, -1, -2, -3, -4
TV_MAX_NODES = 32
TV_MAX_CANDIDATE = 256
TV_LOOKUP_MAX_ORDER = 64
TV_LAYER_ATTN, TV_LAYER_RECUR, TV_LAYER_DELTA = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtreeverify.so")
_lib = None

# every symbol include/treeverify.h declares
SYMBOLS = ("tv_create", "tv_destroy", "tv_last_error", "tv_bind", "tv_set_history",
           "tv_set_modifiers", "tv_set_sampling", "tv_prefill", "tv_prefill_dense", "tv_verify_tree", "tv_verify_trees",
           "tv_accept_walk", "tv_commit", "tv_round", "tv_ctx_len", "tv_profile_enable",
           "tv_profile_reset", "tv_profile_get", "tv_linear", "tv_head_top2", "tv_pack_weight",
           "tv_staircut", "tv_residual_round", "tv_lookup_draft", "tv_attention", "tv_rope_kv",
           "tv_resid_norm", "tv_recur_tree", "tv_recur_commit", "tv_gather_kv", "tv_linear_noalloc",
           "tv_prices_create", "tv_prices_destroy", "tv_prices_class", "tv_prices_table", "tv_prices_observe")


class TVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int), ("hidden", ctypes.c_int), ("n_qhead", ctypes.c_int),
                ("n_kvhead", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int),
                ("vocab", ctypes.c_int), ("layer_kind", ctypes.POINTER(ctypes.c_int)),
                ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("max_ctx", ctypes.c_int), ("max_req", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m greedy_draft_tree_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sig = {
        "tv_create": ([ctypes.POINTER(_Desc), P, ctypes.POINTER(P)], I),
        "tv_destroy": ([P], None),
        "tv_last_error": ([P], ctypes.c_char_p),
        "tv_bind": ([P, ctypes.c_char_p, P, S], I),
        "tv_set_history": ([P, I, P, I, I], I),
        "tv_set_modifiers": ([P, I, F, P, P, I, P], I),
        "tv_set_sampling": ([P, I, F, ctypes.c_uint64], I),
        "tv_prefill": ([P, I, P, I, P], I),
        "tv_prefill_dense": ([P, I, P, I, I, P], I),
        "tv_verify_tree": ([P, I, P, P, I, P, P, P], I),
        "tv_verify_trees": ([P, I, P, P, P, P, P, P, P], I),
        "tv_accept_walk": ([P, P, P, I, P, P, P, P], I),
        "tv_commit": ([P, I, P, I], I),
        "tv_round": ([P, I, P, P, I, P, P, P, P, P, P, P], I),
        "tv_ctx_len": ([P, I], I),
        "tv_profile_enable": ([P, I, ctypes.c_char_p], I),
        "tv_profile_reset": ([P], I),
        "tv_profile_get": ([P, ctypes.c_char_p, P, P], I),
        "tv_linear": ([P, P, P, I, I, I, P, I], I),
        "tv_head_top2": ([P, P, I, P, P, P], I),
        "tv_pack_weight": ([P, P, I, I], I),
        "tv_staircut": ([P, P, P, I, P, P, F, F, P, P, P], I),
        "tv_residual_round": ([P, I, P, P, I, P, F, P, P, P, P, P], I),
        "tv_lookup_draft": ([P, I, I, I, I, I, F, P, P, P, P, P, P, P], I),
        "tv_attention": ([P, P, P, P, I, I, P, I, P], I),
        "tv_rope_kv": ([P, P, I, I, P, I, P, P, P, I], I),
        "tv_resid_norm": ([P, P, I, I, P, P, P], I),
        "tv_recur_tree": ([P, I, P, I, P, I, P, P, P, P, P], I),
        "tv_recur_commit": ([P, P, P, P, P, P, I], I),
        "tv_gather_kv": ([P, P, P, I, I, P, I], I),
        "tv_linear_noalloc": ([P, P, I, I, I, P, I, P], I),
        "tv_prices_create": ([P, P, P, P, I, I, ctypes.c_double, ctypes.c_double, ctypes.POINTER(P)], I),
        "tv_prices_destroy": ([P], None),
        "tv_prices_class": ([P, I, P, P], I),
        "tv_prices_table": ([P, I, I, P], I),
        "tv_prices_observe": ([P, I, I, I, ctypes.c_double], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def exported_symbols() -> Dict[str, bool]:
    lib = load_library()
    return {s: hasattr(lib, s) for s in SYMBOLS}


def _i32(a) -> np.ndarray:
    if type(a) is np.ndarray and a.dtype == np.int32 and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray) -> int:
    """Address of an array's data (ctypes passes an int as void*)."""
    return a.__array_interface__["data"][0]


def _dtype_name(t) -> str:
    return str(getattr(t, "dtype", None)).replace("torch.", "")


def check_device_tensor(t, what: str, dtype: Optional[str] = None, min_numel: int = 0,
                        shape: Optional[Tuple[int, ...]] = None) -> None:
    """Raise ValueError unless ``t`` is a contiguous device tensor of ``dtype``
    ("float32", "bfloat16") with at least ``min_numel`` elements (or exactly
    ``shape``).  The library writes through the raw pointer, so a tensor of
    the wrong element size, on the host or too small would be written past
    its end on the device; every entry point checks before the call."""
    if dtype is not None and _dtype_name(t) != dtype:
        raise ValueError(f"{what}: dtype {_dtype_name(t)}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{what}: tensor must be on the GPU")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() < min_numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {min_numel} needed")


def _logits_ptr(logits, rows: int, vocab: int, what: str):
    """Device address of an fp32 logits buffer with room for [rows, vocab]
    (None passes NULL: the library's own scratch)."""
    if logits is None:
        return None
    check_device_tensor(logits, f"{what}: logits", "float32", rows * vocab)
    return logits.data_ptr()


def linear_noalloc(x, w, y, stream: Optional[int] = None) -> None:
    """tv_linear_noalloc: y = x w^T on static library scratch, no context and
    no allocation; only enqueues on ``stream`` (default: torch's current
    stream, passed by the caller as an int handle)."""
    lib = _lib if _lib is not None else load_library()
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("linear_noalloc: x and w must be matrices")
    M, K = x.shape
    N = w.shape[0]
    check_device_tensor(x, "linear_noalloc: x", "bfloat16")
    check_device_tensor(w, "linear_noalloc: w", "bfloat16", shape=(N, K))
    if _dtype_name(y) not in ("bfloat16", "float32"):
        raise ValueError(f"linear_noalloc: y dtype {_dtype_name(y)}, expected bfloat16 or float32")
    check_device_tensor(y, "linear_noalloc: y", shape=(M, N))
    rc = lib.tv_linear_noalloc(x.data_ptr(), w.data_ptr(), M, N, K, y.data_ptr(),
                               1 if _dtype_name(y) == "float32" else 0, ctypes.c_void_p(stream or 0))
    if rc != TV_OK:
        msg = lib.tv_last_error(None)
        raise TVError(rc, f"tv_linear_noalloc: {msg.decode() if msg else ''}")


# output buffers of accept_walk, reused across calls (results are copied out)
_walk_path = np.zeros(TV_MAX_NODES, np.int32)
_walk_emit = np.zeros(TV_MAX_NODES, np.int32)
_walk_len = (ctypes.c_int32 * 2)()
_walk_ptrs = (_ptr(_walk_path), _ptr(_walk_emit), ctypes.addressof(_walk_len),
              ctypes.addressof(_walk_len) + 4)


def accept_walk(parents: Sequence[int], tokens: Sequence[int], argmax: Sequence[int]
                ) -> Tuple[list, list]:
    """tv_accept_walk: (path node ids, emitted tokens)."""
    lib = _lib if _lib is not None else load_library()
    p, t, a = _i32(parents), _i32(tokens), _i32(argmax)
    n = len(p)
    if n > TV_MAX_NODES or len(t) != n or len(a) < n:
        raise TVError(TV_EINVAL, "tv_accept_walk: bad tree size")
    pp, pe, pl, pn = _walk_ptrs
    rc = lib.tv_accept_walk(_ptr(p), _ptr(t), _ptr(a), n, pp, pl, pe, pn)
    if rc != TV_OK:
        raise TVError(rc, "tv_accept_walk: invalid tree")
    return _walk_path[:_walk_len[0]].tolist(), _walk_emit[:_walk_len[1]].tolist()


class TreeVerifier:
    """One tv_ctx.  Tensors passed to ``bind`` must stay alive while bound."""

    def __init__(self, n_layer: int, hidden: int, n_qhead: int, n_kvhead: int, head_dim: int,
                 ffn: int, vocab: int, layer_kind: Sequence[int], max_ctx: int, max_req: int = 1,
                 eps: float = 1e-6, rope_theta: float = 1e4, stream: Optional[int] = None):
        self.lib = load_library()
        self._kinds = (ctypes.c_int * n_layer)(*[int(k) for k in layer_kind])
        d = _Desc(n_layer, hidden, n_qhead, n_kvhead, head_dim, ffn, vocab, self._kinds,
                  eps, rope_theta, max_ctx, max_req)
        self.vocab, self.max_ctx, self.max_req = vocab, max_ctx, max_req
        self.hidden = hidden
        self.n_qhead, self.n_kvhead, self.head_dim = n_qhead, n_kvhead, head_dim
        # per-call result buffers of tv_verify_tree (copied out on return)
        self._am = np.zeros(TV_MAX_NODES, np.int32)
        self._gap = np.zeros(TV_MAX_NODES, np.float32)
        self._am_ptr, self._gap_ptr = _ptr(self._am), _ptr(self._gap)
        self._path = np.zeros(TV_MAX_NODES, np.int32)
        self._emit = np.zeros(TV_MAX_NODES, np.int32)
        self._lens = (ctypes.c_int32 * 2)()
        self._path_ptr, self._emit_ptr = _ptr(self._path), _ptr(self._emit)
        self._lens_ptr = ctypes.addressof(self._lens)
        h = ctypes.c_void_p()
        rc = self.lib.tv_create(ctypes.byref(d), ctypes.c_void_p(stream or 0), ctypes.byref(h))
        if rc != TV_OK:
            raise TVError(rc, "tv_create failed")
        self.h = h
        self._keep = {}

    @classmethod
    def for_shape(cls, shape, max_ctx: int, max_req: int = 1, stream: Optional[int] = None):
        return cls(shape.n_layer, shape.hidden, shape.n_qhead, shape.n_kvhead, shape.head_dim,
                   shape.ffn, shape.vocab, shape.kinds, max_ctx, max_req, shape.eps,
                   shape.rope_theta, stream)

    def _check(self, rc: int, what: str):
        if rc != TV_OK:
            msg = self.lib.tv_last_error(self.h)
            raise TVError(rc, f"{what}: {msg.decode() if msg else ''}")

    def close(self):
        if getattr(self, "h", None):
            self.lib.tv_destroy(self.h)
            self.h = None
            self._keep.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def bind(self, name: str, tensor) -> None:
        """tv_bind with a contiguous device tensor."""
        check_device_tensor(tensor, name)
        nbytes = tensor.numel() * tensor.element_size()
        self._check(self.lib.tv_bind(self.h, name.encode(), ctypes.c_void_p(tensor.data_ptr()),
                                     nbytes), f"tv_bind({name})")
        self._keep[name] = tensor

    def set_history(self, req: int, ids: Sequence[int], ctx_len: int) -> None:
        a = _i32(ids)
        self._check(self.lib.tv_set_history(self.h, req, _ptr(a) if a.size else None, int(a.size),
                                            int(ctx_len)), "tv_set_history")

    def set_modifiers(self, req: int, rep_penalty: float = 1.0, bias_ids=(), bias_vals=(),
                      allow_bits: Optional[np.ndarray] = None) -> None:
        ids = _i32(bias_ids)
        vals = np.ascontiguousarray(np.asarray(bias_vals, dtype=np.float32))
        bits = None if allow_bits is None else np.ascontiguousarray(allow_bits, dtype=np.uint32)
        self._check(self.lib.tv_set_modifiers(
            self.h, req, float(rep_penalty), _ptr(ids) if ids.size else None,
            _ptr(vals) if vals.size else None, int(ids.size),
            _ptr(bits) if bits is not None else None), "tv_set_modifiers")

    def set_sampling(self, req: int, temperature: float, seed: int = 0) -> None:
        """tv_set_sampling: temperature 0 is greedy."""
        self._check(self.lib.tv_set_sampling(self.h, req, float(temperature),
                                             int(seed) & 0xFFFFFFFFFFFFFFFF), "tv_set_sampling")

    def prefill(self, req: int, tokens: Sequence[int]) -> int:
        t = _i32(tokens)
        out = ctypes.c_int32(0)
        self._check(self.lib.tv_prefill(self.h, req, _ptr(t), int(t.size), ctypes.byref(out)),
                    "tv_prefill")
        return int(out.value)

    def prefill_dense(self, req: int, tokens: Sequence[int], chunk: int = 512) -> int:
        """tv_prefill_dense: the prompt on the dense prefill kernels, chunked
        on the grid of multiples of `chunk`; returns the last row's token."""
        t = _i32(tokens)
        out = ctypes.c_int32(0)
        self._check(self.lib.tv_prefill_dense(self.h, req, _ptr(t), int(t.size), int(chunk), ctypes.byref(out)),
                    "tv_prefill_dense")
        return int(out.value)

    def verify_tree(self, req: int, parents, tokens, logits=None):
        """tv_verify_tree -> (argmax int32 [n], gap_ulps float32 [n]).
        ``logits``: optional device fp32 tensor with room for [n, vocab]."""
        p, t = _i32(parents), _i32(tokens)
        n = int(p.size)
        lp = _logits_ptr(logits, n, self.vocab, "verify_tree")
        rc = self.lib.tv_verify_tree(self.h, req, _ptr(p), _ptr(t), n, lp, self._am_ptr, self._gap_ptr)
        if rc != TV_OK:
            self._check(rc, "tv_verify_tree")
        return self._am[:n].copy(), self._gap[:n].copy()

    def verify_trees(self, reqs: Sequence[int], parents: Sequence, tokens: Sequence, logits=None):
        """tv_verify_trees: rows request after request."""
        k = len(reqs)
        ps = [_i32(p) for p in parents]
        ts = [_i32(t) for t in tokens]
        ns = np.array([p.size for p in ps], np.int32)
        total = int(ns.sum())
        rq = _i32(reqs)
        pp = (ctypes.c_void_p * k)(*[p.ctypes.data for p in ps])
        tp = (ctypes.c_void_p * k)(*[t.ctypes.data for t in ts])
        am = np.zeros(max(total, 1), np.int32)
        gap = np.zeros(max(total, 1), np.float32)
        lp = _logits_ptr(logits, total, self.vocab, "verify_trees")
        self._check(self.lib.tv_verify_trees(self.h, k, _ptr(rq), ctypes.cast(pp, ctypes.c_void_p),
                                             ctypes.cast(tp, ctypes.c_void_p), _ptr(ns), lp,
                                             _ptr(am), _ptr(gap)), "tv_verify_trees")
        return am[:total], gap[:total]

    def commit(self, req: int, path: Sequence[int]) -> None:
        p = _i32(path)
        rc = self.lib.tv_commit(self.h, req, _ptr(p), int(p.size))
        if rc != TV_OK:
            self._check(rc, "tv_commit")

    def round(self, req: int, parents, tokens, logits=None):
        """tv_round: verify, accept walk and commit in one call ->
        (argmax, gap, path, emitted)."""
        p, t = _i32(parents), _i32(tokens)
        n = int(p.size)
        lp = _logits_ptr(logits, n, self.vocab, "round")
        rc = self.lib.tv_round(self.h, req, _ptr(p), _ptr(t), n, lp, self._am_ptr, self._gap_ptr,
                               self._path_ptr, self._lens_ptr, self._emit_ptr, self._lens_ptr + 4)
        if rc != TV_OK:
            self._check(rc, "tv_round")
        return (self._am[:n].copy(), self._gap[:n].copy(), self._path[:self._lens[0]].tolist(),
                self._emit[:self._lens[1]].tolist())

    def residual_round(self, req: int, parents, tokens, temperature: float, uniforms, logits=None):
        """tv_residual_round: (path, emitted) of one residual-sampling round;
        uniforms[d] is the uniform of depth d."""
        p, t = _i32(parents), _i32(tokens)
        n = len(p)
        u = np.ascontiguousarray(np.asarray(uniforms, dtype=np.float64))
        if u.shape[0] < n:
            raise TVError(-1, "tv_residual_round: one uniform per depth (at least n_nodes)")
        lp = _logits_ptr(logits, n, self.vocab, "residual_round")
        rc = self.lib.tv_residual_round(self.h, req, _ptr(p), _ptr(t), n, lp, float(temperature), _ptr(u),
                                        _ptr(self._path), ctypes.addressof(self._lens), _ptr(self._emit),
                                        ctypes.addressof(self._lens) + 4)
        self._check(rc, "tv_residual_round")
        return self._path[:self._lens[0]].tolist(), self._emit[:self._lens[1]].tolist()

    def ctx_len(self, req: int) -> int:
        rc = self.lib.tv_ctx_len(self.h, req)
        if rc < 0:
            self._check(rc, "tv_ctx_len")
        return rc

    def linear(self, x, w, y) -> None:
        """tv_linear: y = x w^T (bf16 out if y is bf16, fp32 sums if y is fp32);
        w must have been packed with pack_weight."""
        if x.dim() != 2 or w.dim() != 2:
            raise ValueError("linear: x and w must be matrices")
        M, K = x.shape
        N = w.shape[0]
        check_device_tensor(x, "linear: x", "bfloat16")
        check_device_tensor(w, "linear: w", "bfloat16", shape=(N, K))
        if _dtype_name(y) not in ("bfloat16", "float32"):
            raise ValueError(f"linear: y dtype {_dtype_name(y)}, expected bfloat16 or float32")
        check_device_tensor(y, "linear: y", shape=(M, N))
        fp32 = 1 if _dtype_name(y) == "float32" else 0
        self._check(self.lib.tv_linear(self.h, ctypes.c_void_p(x.data_ptr()),
                                       ctypes.c_void_p(w.data_ptr()), M, N, K,
                                       ctypes.c_void_p(y.data_ptr()), fp32), "tv_linear")

    def pack_weight(self, w) -> None:
        """tv_pack_weight: rearrange a row-major [N, K] bf16 tensor in place."""
        if w.dim() != 2:
            raise ValueError("pack_weight: w must be a matrix")
        check_device_tensor(w, "pack_weight: w", "bfloat16")
        N, K = w.shape
        self._check(self.lib.tv_pack_weight(self.h, ctypes.c_void_p(w.data_ptr()), N, K),
                    "tv_pack_weight")

    def head_top2(self, x, logits):
        """tv_head_top2 on x [M, hidden] bf16 -> (argmax, gap)."""
        if x.dim() != 2 or not (1 <= x.shape[0] <= TV_MAX_NODES):
            raise ValueError("head_top2: x must be [M, hidden] with 1 <= M <= 32")
        M = x.shape[0]
        check_device_tensor(x, "head_top2: x", "bfloat16", shape=(M, self.hidden))
        check_device_tensor(logits, "head_top2: logits", "float32", M * self.vocab)
        am = np.zeros(M, np.int32)
        gap = np.zeros(M, np.float32)
        self._check(self.lib.tv_head_top2(self.h, ctypes.c_void_p(x.data_ptr()), M,
                                          ctypes.c_void_p(logits.data_ptr()), _ptr(am), _ptr(gap)),
                    "tv_head_top2")
        return am, gap

    # ------------------------------------------------ kernel-level calls

    def _partials(self, part, splits: int, rows: int, cols: int, what: str) -> int:
        """Device address of split-K partials for `rows` rows and `cols`
        columns in the library's layout (128-column blocks of 32 rows)."""
        need = ((cols + 127) // 128) * int(splits) * 4096
        if not (1 <= rows <= TV_MAX_NODES):
            raise ValueError(f"{what}: {rows} rows, 1..32 supported")
        check_device_tensor(part, f"{what}: partials", "float32", need)
        return part.data_ptr()

    def attention(self, q, k_cache, v_cache, ctx_len: int, parents, out) -> None:
        """tv_attention: tree-masked attention of the tree's rows."""
        p = _i32(parents)
        n, QD = int(p.size), self.n_qhead * self.head_dim
        check_device_tensor(q, "attention: q", "bfloat16", shape=(n, QD))
        check_device_tensor(out, "attention: out", "bfloat16", shape=(n, QD))
        check_device_tensor(k_cache, "attention: k_cache", "bfloat16")
        check_device_tensor(v_cache, "attention: v_cache", "bfloat16", shape=tuple(k_cache.shape))
        kvh, cap, d = k_cache.shape
        if (kvh, d) != (self.n_kvhead, self.head_dim):
            raise ValueError("attention: cache shape does not match the model")
        self._check(self.lib.tv_attention(self.h, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), int(cap),
                                          int(ctx_len), _ptr(p), n, out.data_ptr()), "tv_attention")

    def rope_kv(self, part, splits: int, depth, ctx_len: int, q_out, k_cache, v_cache) -> None:
        """tv_rope_kv: finish the QKV partials, rotate q and k, write the cache."""
        dep = _i32(depth)
        n = int(dep.size)
        cols = (self.n_qhead + 2 * self.n_kvhead) * self.head_dim
        pp = self._partials(part, splits, n, cols, "rope_kv")
        check_device_tensor(q_out, "rope_kv: q_out", "bfloat16", shape=(n, self.n_qhead * self.head_dim))
        check_device_tensor(k_cache, "rope_kv: k_cache", "bfloat16")
        check_device_tensor(v_cache, "rope_kv: v_cache", "bfloat16", shape=tuple(k_cache.shape))
        kvh, cap, d = k_cache.shape
        if (kvh, d) != (self.n_kvhead, self.head_dim):
            raise ValueError("rope_kv: cache shape does not match the model")
        self._check(self.lib.tv_rope_kv(self.h, pp, int(splits), n, _ptr(dep), int(ctx_len), q_out.data_ptr(),
                                        k_cache.data_ptr(), v_cache.data_ptr(), int(cap)), "tv_rope_kv")

    def resid_norm(self, part, splits: int, x, w, y) -> None:
        """tv_resid_norm: x += bf16(partial sums); y = RMSNorm(x) * w."""
        n = int(x.shape[0])
        pp = self._partials(part, splits, n, self.hidden, "resid_norm")
        check_device_tensor(x, "resid_norm: x", "bfloat16", shape=(n, self.hidden))
        check_device_tensor(y, "resid_norm: y", "bfloat16", shape=(n, self.hidden))
        check_device_tensor(w, "resid_norm: w", "bfloat16", shape=(self.hidden,))
        self._check(self.lib.tv_resid_norm(self.h, pp, int(splits), n, x.data_ptr(), w.data_ptr(), y.data_ptr()),
                    "tv_resid_norm")

    def recur_tree(self, kind: int, part, splits: int, parents, state, out, save_k, save_v, save_gc) -> None:
        """tv_recur_tree: recurrent read-out of a tree and the saves for a commit."""
        p = _i32(parents)
        n = int(p.size)
        QH, D = self.n_qhead, self.head_dim
        cols = 3 * QH * D + (2 if kind == TV_LAYER_DELTA else 1) * QH
        pp = self._partials(part, splits, n, cols, "recur_tree")
        check_device_tensor(state, "recur_tree: state", "float32", shape=(QH, D, D))
        check_device_tensor(out, "recur_tree: out", "bfloat16", shape=(n, QH * D))
        check_device_tensor(save_k, "recur_tree: save_k", "bfloat16", shape=(TV_MAX_NODES, QH, D))
        check_device_tensor(save_v, "recur_tree: save_v", "float32", shape=(TV_MAX_NODES, QH, D))
        check_device_tensor(save_gc, "recur_tree: save_gc", "float32", shape=(TV_MAX_NODES, QH))
        self._check(self.lib.tv_recur_tree(self.h, int(kind), pp, int(splits), _ptr(p), n, state.data_ptr(),
                                           out.data_ptr(), save_k.data_ptr(), save_v.data_ptr(),
                                           save_gc.data_ptr()), "tv_recur_tree")

    def recur_commit(self, state, save_k, save_v, save_gc, path) -> None:
        """tv_recur_commit: the state after `path` from tv_recur_tree's saves."""
        pa = _i32(path)
        QH, D = self.n_qhead, self.head_dim
        check_device_tensor(state, "recur_commit: state", "float32", shape=(QH, D, D))
        check_device_tensor(save_k, "recur_commit: save_k", "bfloat16", shape=(TV_MAX_NODES, QH, D))
        check_device_tensor(save_v, "recur_commit: save_v", "float32", shape=(TV_MAX_NODES, QH, D))
        check_device_tensor(save_gc, "recur_commit: save_gc", "float32", shape=(TV_MAX_NODES, QH))
        self._check(self.lib.tv_recur_commit(self.h, state.data_ptr(), save_k.data_ptr(), save_v.data_ptr(),
                                             save_gc.data_ptr(), _ptr(pa), int(pa.size)), "tv_recur_commit")

    def gather_kv(self, k_cache, v_cache, ctx_len: int, path) -> None:
        """tv_gather_kv: cache slot ctx_len + path[d] -> ctx_len + d."""
        pa = _i32(path)
        check_device_tensor(k_cache, "gather_kv: k_cache", "bfloat16")
        check_device_tensor(v_cache, "gather_kv: v_cache", "bfloat16", shape=tuple(k_cache.shape))
        kvh, cap, d = k_cache.shape
        if (kvh, d) != (self.n_kvhead, self.head_dim):
            raise ValueError("gather_kv: cache shape does not match the model")
        self._check(self.lib.tv_gather_kv(self.h, k_cache.data_ptr(), v_cache.data_ptr(), int(cap), int(ctx_len),
                                          _ptr(pa), int(pa.size)), "tv_gather_kv")

    def profile_enable(self, on: bool = True, only_prefix: str = "") -> None:
        self._check(self.lib.tv_profile_enable(self.h, int(on), only_prefix.encode()),
                    "tv_profile_enable")

    def profile_reset(self) -> None:
        self._check(self.lib.tv_profile_reset(self.h), "tv_profile_reset")

    def profile_get(self, prefix: str) -> Tuple[float, int]:
        ms, cnt = ctypes.c_double(0), ctypes.c_int(0)
        self._check(self.lib.tv_profile_get(self.h, prefix.encode(), ctypes.byref(ms),
                                            ctypes.byref(cnt)), "tv_profile_get")
        return ms.value, cnt.value
