"""Benchmark: ms per tree verify and achieved HBM GB/s at 8/16/24/32 nodes.

One step is one pass of the whole hot path for each tree size n in
{8, 16, 24, 32}: tree verify (one target-model forward over the tree against
the KV cache, fp32 logits, argmax and top-2 gap per node), the greedy accept
walk, and the commit of the accepted path's KV rows.  After each commit the
request's context is reset to ``ctx`` (host metadata only), so every round
runs at the same context length.  The draft trees carry the model's own
greedy tokens along their spine (learned in warm-up), so the accept walk
takes the whole spine and the commit moves real rows; branches are uniform
ids.

Inputs are synthetic and resident in HBM before timing: N(0, 0.02) bf16
weights drawn on the device, an N(0, 1) bf16 KV cache of ``ctx`` rows.

``value`` is the whole step's algorithmic HBM bytes (weights once per
verify, KV read, tree KV write, logits write, committed rows moved) divided
by its wall time.  ``roofline`` reports the dominant kernel (the fp32 head)
timed with HIP events on the library's stream during the timed region.
``cpu_baseline`` times the CPU oracle on the same trees.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
NS = (8, 16, 24, 32)
MIN_CPU_S = 10.0     # the CPU baseline repeats its sample for at least this long


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c1", choices=["c1", "c2"])
    ap.add_argument("--ctx", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", default="full",
                    help="'full' = the same four trees; 'n8' = one 8-node tree")
    ap.add_argument("--kernel-breakdown", action="store_true",
                    help="add per-kernel event timings (an extra untimed pass)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device copy first (calibrates HBM byte counters)")
    return ap.parse_args()


def model_bytes(shape, n, ctx, path_len):
    """Algorithmic HBM bytes of one verify + commit (see module docstring)."""
    H, V, F = shape.hidden, shape.vocab, shape.ffn
    D, QH, KVH = shape.head_dim, shape.n_qhead, shape.n_kvhead
    b = 0
    b += n * H * 2                                  # embedding rows
    for kind in shape.kinds:
        b += 2 * H * 2                              # two norm vectors
        b += shape.qkv_rows * H * 2                 # wqkv
        b += H * QH * D * 2                         # wo
        b += 3 * F * H * 2                          # wg, wu, wd
        b += 2 * ctx * KVH * D * 2                  # cache K and V read
        b += 2 * n * KVH * D * 2                    # tree K and V written
        b += 2 * 2 * path_len * KVH * D * 2         # committed rows read + written
    b += H * 2 + V * H * 2                          # final norm, head
    b += n * V * 4                                  # fp32 logits
    return b


def committed_traffic():
    """Per-launch HBM bytes of the head kernel from the committed rocprofv3
    counter summary, if the kernel source it was taken on is unchanged."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    summ = os.path.join(here, "profiles", "gemm_head_c1_layer_ctx1024_counters.md")
    src = os.path.join(here, "greedy_draft_tree_amd", "csrc", "tv_kernels.hip")
    if not os.path.exists(summ):
        return None
    fields = {}
    for line in open(summ):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel source sha256") != sha:
        return None
    try:
        return float(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def head_bytes(shape, n):
    return shape.vocab * shape.hidden * 2 + n * shape.vocab * 4 + n * shape.hidden * 2


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(a verify does not shard: see the design notes on multi-GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import workloads

    shape = synth.C1 if a.config == "c1" else synth.C2
    ctx = a.ctx
    torch.cuda.init()
    if a.copy_probe:
        src_t = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst_t = torch.empty_like(src_t)
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t
    print(f"[bench] building {shape.name} ctx={ctx}", file=sys.stderr, flush=True)
    want_cpu = not a.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0
    wl = workloads.build(shape, max_ctx=ctx + 64, max_req=1, weight_device="cuda",
                         host_copy=want_cpu)
    kv = workloads.load_context(wl, 0, ctx, seed=3)
    tv = wl.tv
    from greedy_draft_tree_amd import accept_walk

    # trees: spine carries the model's own greedy tokens (learned in warm-up)
    trees = {}
    for n in NS:
        parents = synth.spine_tree(n, 4)
        tokens = synth.tree_tokens(parents, shape.vocab, 5 + n, root_token=17)
        spine = synth.spine_nodes(parents)
        for d in range(len(spine) - 1):
            am, _ = tv.verify_tree(0, parents, tokens)
            want = int(am[spine[d]])
            sib = {int(tokens[j]) for j in range(1, n) if parents[j] == parents[spine[d + 1]]
                   and j != spine[d + 1]}
            if want in sib:
                break
            tokens[spine[d + 1]] = want
        trees[n] = (parents, tokens)
    print("[bench] trees ready", file=sys.stderr, flush=True)

    def round_(n):
        parents, tokens = trees[n]
        am, _ = tv.verify_tree(0, parents, tokens, logits=wl.logits)
        path, _ = accept_walk(parents, tokens, am)
        tv.commit(0, path)
        tv.set_history(0, [], ctx)
        return len(path)

    for _ in range(a.warmup):
        for n in NS:
            round_(n)
    path_lens = {n: round_(n) for n in NS}

    tv.profile_reset()
    tv.profile_enable(True, "gemm_head")
    per_n = {n: [] for n in NS}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for n in NS:
            s = time.perf_counter()
            round_(n)
            per_n[n].append(time.perf_counter() - s)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    head_ms, head_cnt = tv.profile_get("gemm_head")
    tv.profile_enable(False)

    step_bytes = sum(model_bytes(shape, n, ctx, path_lens[n]) for n in NS)
    value = step_bytes * a.steps / total / 1e9
    per = {}
    for n in NS:
        ms = float(np.median(per_n[n]) * 1e3)
        by = model_bytes(shape, n, ctx, path_lens[n])
        per[str(n)] = {"ms_median": round(ms, 4), "ms_min": round(float(np.min(per_n[n]) * 1e3), 4),
                       "GBps": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / HBM_PEAK_GBS, 4),
                       "rows_per_s": round(n / ms * 1e3, 1), "bytes": by, "path_len": path_lens[n]}
    ratio = per["16"]["ms_median"] / per["8"]["ms_median"]
    head_avg_ms = head_ms / max(head_cnt, 1)
    hb = np.mean([head_bytes(shape, n) for n in NS])
    achieved = hb / (head_avg_ms * 1e-3) / 1e9

    kernels = None
    if a.kernel_breakdown:
        tv.profile_reset()
        tv.profile_enable(True, "")
        for _ in range(5):
            for n in NS:
                round_(n)
        kernels = {}
        for k in ("embed_norm", "resid_norm", "gemm_qkv", "rope_kv", "attn_combine", "attn", "gemm_o",
                  "gemm_gateup", "gemm_down", "gemm_gate", "recur_tree", "gemm_head", "top2", "commit_kv",
                  "commit_state"):
            ms, cnt = tv.profile_get(k)
            if cnt:
                kernels[k] = {"avg_us": round(ms / cnt * 1e3, 2), "launches": cnt}
        if "attn" in kernels and "attn_combine" in kernels:
            ms, cnt = tv.profile_get("attn")
            ms2, cnt2 = tv.profile_get("attn_combine")
            kernels["attn"] = {"avg_us": round((ms - ms2) / max(cnt - cnt2, 1) * 1e3, 2),
                               "launches": cnt - cnt2}
        tv.profile_enable(False)

    cpu = None
    if want_cpu:
        cpu = cpu_baseline(shape, wl, kv, ctx, trees, a.cpu_sample)

    out = {
        "metric": "ms per tree verify + achieved HBM GB/s at 8/16/24/32 nodes, 1k ctx, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(total / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: {shape.n_layer} x (hidden {shape.hidden}, "
                               f"{shape.n_qhead}q/{shape.n_kvhead}kv heads x {shape.head_dim}, "
                               f"SwiGLU {shape.ffn}) + fp32 head V={shape.vocab}; KV cache {ctx} rows; "
                               f"one step = verify+accept+commit of trees n=8,16,24,32",
                   "ctx": ctx, "tree_nodes": list(NS), "step_bytes": step_bytes},
        "per_n": per,
        "ratio_16_over_8": round(ratio, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": committed_traffic() if a.config == "c1" else None,
                     "kernel": "gemm_head (k_gemm<EPI_HEAD>)", "avg_us": round(head_avg_ms * 1e3, 2),
                     "bytes_per_launch": int(hb), "launches": head_cnt},
        "cpu_baseline": cpu,
    }
    if kernels:
        out["kernels"] = kernels
    print(json.dumps(out), flush=True)


def cpu_baseline(shape, wl, kv, ctx, trees, sample):
    """The CPU oracle (brute-force tree scorer) on the same trees."""
    import torch
    import oracle
    w_cpu = wl.host_weights
    kv_cpu = {k: v[:, :ctx].cpu() for k, v in kv.items()}
    orc = oracle.Oracle(shape, w_cpu)
    seq = orc.new_seq(cap=ctx + 40, kv=kv_cpu, ctx_len=ctx)
    ns = NS if sample == "full" else (8,)
    t0 = time.perf_counter()
    by, trees_done, passes = 0, 0, 0
    while True:   # whole passes over the sample until at least MIN_CPU_S seconds
        for n in ns:
            parents, tokens = trees[n]
            orc.tree_scores(seq, parents, tokens)
            by += model_bytes(shape, n, ctx, 1)
            trees_done += 1
        passes += 1
        print(f"[bench] cpu baseline pass {passes} done", file=sys.stderr, flush=True)
        if time.perf_counter() - t0 >= MIN_CPU_S:
            break
    dt = time.perf_counter() - t0
    return {"value": round(by / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.get_threads(),
            "kind": "oracle",
            "sample": f"brute-force oracle tree scores for n={list(ns)} on {shape.name}, ctx {ctx}, "
                      f"{passes} pass(es) ({dt:.1f} s; {dt / trees_done * 1e3:.0f} ms per tree on average)"}


if __name__ == "__main__":
    main()
