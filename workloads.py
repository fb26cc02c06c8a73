"""Synthetic workloads on the device, bound to a TreeVerifier.

Shared by the GPU tests, ``__graft_entry__.smoke`` and ``bench.py``.  Inputs
come from ``synth`` (seeded, no arithmetic of the method); this module only
moves them to the device and binds them.  It never imports the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

import synth
from greedy_draft_tree_amd import TreeVerifier


@dataclasses.dataclass
class Workload:
    shape: synth.ModelShape
    tv: TreeVerifier
    weights: Dict[str, torch.Tensor]           # device bf16 (matrices packed in place by bind)
    kv: Dict[int, Dict]                        # req -> {(layer, 'k'|'v'): device tensor}
    states: Dict[int, Dict]                    # req -> {layer: device fp32 [QH, D, D]}
    max_ctx: int
    logits: torch.Tensor                       # device fp32 [32, V]
    host_weights: Optional[Dict[str, torch.Tensor]] = None  # row-major CPU copies, taken before bind


def build(shape: synth.ModelShape, max_ctx: int, max_req: int = 1, weight_seed: int = 0,
          weight_device: str = "cpu", weights: Optional[Dict[str, torch.Tensor]] = None,
          device: str = "cuda", host_copy: bool = False) -> Workload:
    """Allocate and bind weights (drawn on ``weight_device``), zeroed KV caches
    of ``max_ctx`` rows and zero recurrent states for ``max_req`` requests.
    Binding rearranges the weight matrices in place; ``host_copy`` keeps
    row-major CPU copies taken before that (for the oracle)."""
    if weights is None:
        w = synth.weights(shape, seed=weight_seed, device=weight_device)
        weights = {k: v.to(device) for k, v in w.items()}
        del w
    host = {k: v.cpu() for k, v in weights.items()} if host_copy else None
    stream = torch.cuda.current_stream().cuda_stream
    tv = TreeVerifier.for_shape(shape, max_ctx=max_ctx, max_req=max_req, stream=stream)
    for k, v in weights.items():
        tv.bind(k, v)
    kv, states = {}, {}
    for r in range(max_req):
        kv[r], states[r] = {}, {}
        for l, kind in enumerate(shape.kinds):
            if kind == synth.ATTN:
                for nm in ("k", "v"):
                    t = torch.zeros((shape.n_kvhead, max_ctx, shape.head_dim), dtype=torch.bfloat16,
                                    device=device)
                    tv.bind(f"req.{r}.layers.{l}.{nm}", t)
                    kv[r][(l, nm)] = t
            else:
                t = torch.zeros((shape.n_qhead, shape.head_dim, shape.head_dim), dtype=torch.float32,
                                device=device)
                tv.bind(f"req.{r}.layers.{l}.state", t)
                states[r][l] = t
    logits = torch.empty((32, shape.vocab), dtype=torch.float32, device=device)
    return Workload(shape, tv, weights, kv, states, max_ctx, logits, host)


def load_context(wl: Workload, req: int, ctx: int, seed: int, history=None,
                 state_seed: Optional[int] = None, src_kv=None, src_states=None):
    """Fill request ``req``'s cache rows [0, ctx) with synthetic N(0,1) rows
    (or ``src_kv``) and its states with N(0,1) (or ``src_states``)."""
    kvs = src_kv if src_kv is not None else synth.kv_cache(wl.shape, ctx, seed, cap=ctx, device="cuda")
    for key, t in wl.kv[req].items():
        t.zero_()
        t[:, :ctx].copy_(kvs[key][:, :ctx])
    if wl.states[req]:
        st = src_states if src_states is not None else synth.state0(
            wl.shape, seed if state_seed is None else state_seed, device="cuda")
        for l, t in wl.states[req].items():
            t.copy_(st[l])
    ids = [] if history is None else list(history)
    wl.tv.set_history(req, ids, ctx)
    torch.cuda.synchronize()
    return kvs
