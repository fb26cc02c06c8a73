"""Benchmark: ms per tree verify and achieved HBM GB/s at 8/16/24/32 nodes.

One step is one pass of the whole hot path for each tree size n in
{8, 16, 24, 32}: tree verify (one target-model forward over the tree against
the KV cache, fp32 logits, argmax and top-2 gap per node), the greedy accept
walk, and the commit of the accepted path's KV rows (and recurrent states).
After each commit the request's context is reset to ``ctx`` (host metadata
only), so every round runs at the same context length.  The draft trees carry
the model's own greedy tokens along their spine (learned in warm-up), so the
accept walk takes the spine and the commit moves real rows; branches are
uniform ids.

Configurations (``--config``; the default c2 is the headline workload):

* c2: 64 decoder layers of width 5120 + fp32 head (about 27B parameters),
  trees n = 8/16/24/32 at ``ctx`` (1024); with no ``--no-extras`` the same
  stack is also timed at the ``--extra-ctx`` contexts (8192), reported as
  extra keys ``ctx<N>``, and one such layer + the head (c1) as the extra key
  ``c1_layer``.
* c1: one 5120-wide decoder layer + fp32 head, trees n = 8/16/24/32.
* c3: the 64-layer hybrid (48 gated-recurrence + 16 attention layers), n = 16.
* c3d: c3 with gated delta-rule (Gated DeltaNet) layers in place of the plain
  gated recurrence, n = 16.
* c4: c2 with two requests of 16 rows each in one joint pass (contexts
  ``ctx`` and ``--ctx2``), score modifiers on both (repetition penalty 1.1,
  64 biased ids, a 50% allow mask) and a drafter that is always wrong, so
  every round commits one token per request.

``--temperature T`` (> 0) makes every request a sampled one (seeded
Gumbel-max draws in the head kernel); the spine then carries the request's
own draws.  The bytes are the same as greedy: the noise is generated, not read.

Inputs are synthetic and resident in HBM before timing: N(0, 0.02) bf16
weights drawn on the device, N(0, 1) bf16 KV caches (and N(0, 1) fp32
recurrent states) of ``ctx`` rows.

``value`` is the whole step's algorithmic HBM bytes (weights once per verify,
KV and state reads, tree KV written, logits written, committed rows and
states moved) divided by its wall time.  ``roofline`` reports the dominant
kernel (the fp32 head for c1; the gate/up projection, which takes the most
time summed over layers, for the stacks) timed with HIP events on the
library's stream during the timed region; ``traffic`` is the kernel's HBM
bytes per launch from the committed rocprofv3 counter summary in profiles/,
reported only while the kernel source matches the one counted.
``cpu_baseline`` times the CPU oracle on one 8-node tree of the same
workload (``--cpu-sample full``: the four trees), repeated for at least 10 s
(c1 and c2).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
NS = (8, 16, 24, 32)
MIN_CPU_S = 10.0     # the CPU baseline repeats its sample for at least this long
ATTN, RECUR, DELTA = 0, 1, 2   # layer kinds (as in synth)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c3d", "c4"])
    ap.add_argument("--ctx", type=int, default=1024)
    ap.add_argument("--ctx2", type=int, default=8192, help="second request's context (c4)")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="> 0: every request samples (seeded Gumbel-max draws); 0 = greedy")
    ap.add_argument("--seed", type=int, default=42, help="sampling seed")
    ap.add_argument("--residual", type=float, default=0.0,
                    help="> 0: every round is a residual-sampling round at this temperature (c1/c2)")
    ap.add_argument("--prices", action="store_true",
                    help="instead of the bench line, print a verify price file (StairCut's stair tables) "
                         "for rows 1..32, chain and tree, at the --price-ctx lengths")
    ap.add_argument("--price-ctx", default="1024,8192,32768")
    ap.add_argument("--lookup", action="store_true",
                    help="host cost per call of the lookup drafter at the --price-ctx lengths (no GPU)")
    ap.add_argument("--prefill", type=int, default=0,
                    help="instead of the bench line, time a dense prefill of this many tokens (one JSON line)")
    ap.add_argument("--chunk", type=int, default=512, help="dense prefill chunk (rows)")
    ap.add_argument("--price-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-ctx", default="8192",
                    help="c2: the same stack also timed at these contexts (extra keys ctx<N>)")
    ap.add_argument("--no-extras", action="store_true",
                    help="c2: skip the extra contexts and the one-layer (c1) extra keys")
    ap.add_argument("--cpu-sample", default="n8",
                    help="'full' = the same four trees; 'n8' = one 8-node tree")
    ap.add_argument("--kernel-breakdown", action="store_true",
                    help="add per-kernel event timings (an extra untimed pass)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device copy first (calibrates HBM byte counters)")
    return ap.parse_args()


def model_bytes(shape, n, ctxs, path_lens, mods=False):
    """Algorithmic HBM bytes of one verify (n rows per request, requests with
    contexts ``ctxs``) and the commits of ``path_lens`` (module docstring)."""
    H, V, F = shape.hidden, shape.vocab, shape.ffn
    D, QH, KVH = shape.head_dim, shape.n_qhead, shape.n_kvhead
    rows = n * len(ctxs)
    b = rows * H * 2                                    # embedding rows
    for kind in shape.kinds:
        b += 2 * H * 2                                  # two norm vectors
        if kind == ATTN:
            b += shape.qkv_rows * H * 2                 # wqkv
            for ctx, pl in zip(ctxs, path_lens):
                b += 2 * ctx * KVH * D * 2              # cache K and V read
                b += 2 * n * KVH * D * 2                # tree K and V written
                b += 2 * 2 * pl * KVH * D * 2           # committed rows read + written
        else:
            b += shape.rqkv_rows * H * 2                # wqkv
            b += (2 if kind == DELTA else 1) * QH * H * 2   # gate (and write-strength) projection
            for _ in ctxs:
                b += QH * D * D * 4                     # state read by the verify
                b += 2 * QH * D * D * 4                 # state read + written by the commit
        b += H * QH * D * 2                             # wo
        b += 3 * F * H * 2                              # wg, wu, wd
    b += H * 2 + V * H * 2                              # final norm, head
    b += rows * V * 4                                   # fp32 logits
    if mods:
        b += len(ctxs) * (V * 4 + 2 * ((V + 31) // 32) * 4)   # bias, allow and history bits
    return b


def committed_traffic(summary):
    """Per-launch HBM bytes of a kernel from its committed rocprofv3 counter
    summary (profiles/<summary>), if the kernel source it was taken on is
    unchanged."""
    here = os.path.dirname(os.path.abspath(__file__))
    summ = os.path.join(here, "profiles", summary)
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


def head_bytes(shape, rows):
    return shape.vocab * shape.hidden * 2 + rows * shape.vocab * 4 + rows * shape.hidden * 2


def gateup_bytes(shape, rows):
    return 2 * shape.ffn * shape.hidden * 2 + rows * shape.hidden * 2


def learn_spine(tv, parents, tokens, req=0):
    """Put the model's own token (the argmax, or a sampled request's draw)
    on each spine node, depth by depth."""
    import synth
    n = len(parents)
    spine = synth.spine_nodes(parents)
    for d in range(len(spine) - 1):
        am, _ = tv.verify_tree(req, parents, tokens)
        want = int(am[spine[d]])
        sib = {int(tokens[j]) for j in range(1, n) if parents[j] == parents[spine[d + 1]]
               and j != spine[d + 1]}
        if want in sib:
            break
        tokens[spine[d + 1]] = want
    return tokens


def make_wrong(parents, tokens, argmax, vocab):
    """Change every node whose token equals its parent's argmax, keeping
    sibling tokens distinct: the walk then accepts nothing past the root."""
    tokens = tokens.copy()
    for j in range(1, len(parents)):
        p = parents[j]
        if tokens[j] == argmax[p]:
            sib = {int(tokens[i]) for i in range(1, len(parents)) if parents[i] == p and i != j}
            t = (int(argmax[p]) + 1) % vocab
            while t in sib or t == argmax[p]:
                t = (t + 1) % vocab
            tokens[j] = t
    return tokens


def build_workload(a, shape, max_ctx, n_req, want_cpu):
    import torch
    import workloads
    print(f"[bench] building {shape.name} (max ctx {max_ctx})", file=sys.stderr, flush=True)
    wl = workloads.build(shape, max_ctx=max_ctx, max_req=n_req, weight_device="cuda", host_copy=want_cpu)
    torch.cuda.synchronize()
    return wl


def setup(a, wl, shape, ns, ctxs, mods_on):
    """Load the contexts (synthetic caches and states), modifiers and
    sampling, and make the trees: the spine carries the model's own tokens
    (learned here), or for the joint config a drafter wrong at every node."""
    import synth
    import workloads
    tv = wl.tv
    n_req = len(ctxs)
    hist, kv = [], None
    for r, ctx in enumerate(ctxs):
        h = synth.uniform_ids(ctx, shape.vocab, 40 + r) if mods_on else []
        kvr = workloads.load_context(wl, r, ctx, seed=3 + r, history=h, state_seed=6)
        if r == 0:
            kv = kvr
        hist.append(h)
    for r in range(n_req):
        if mods_on:
            md = synth.modifiers(shape.vocab, 7 + r)
            tv.set_modifiers(r, md.rep_penalty, md.bias_ids, md.bias_vals, md.allow_bits)
        else:
            tv.set_modifiers(r, 1.0)
        tv.set_sampling(r, a.temperature if a.temperature > 0 else 0.0, a.seed + r)
    trees = {}
    for n in ns:
        per_req = []
        for r in range(n_req):
            parents = synth.spine_tree(n, 4)
            tokens = synth.tree_tokens(parents, shape.vocab, 5 + n + 100 * r, root_token=17 + r)
            if mods_on:
                for _ in range(4):   # a changed token changes its subtree's rows: repeat until stable
                    am, _ = tv.verify_tree(r, parents, tokens)
                    fixed = make_wrong(parents, tokens, am, shape.vocab)
                    if np.array_equal(fixed, tokens):
                        break
                    tokens = fixed
            else:
                tokens = learn_spine(tv, parents, tokens, r)
            per_req.append((parents, tokens))
        trees[n] = per_req
    print(f"[bench] {shape.name} ctx {ctxs}: trees ready", file=sys.stderr, flush=True)
    return hist, kv, trees


def time_rounds(a, wl, shape, ns, ctxs, hist, trees, kern, mods_on):
    """Warm-up, then exactly a.steps steps (every tree size once per step),
    bracketed by device synchronisations; the dominant kernel `kern` is
    timed by HIP events on the library's stream during the timed steps."""
    import torch
    from greedy_draft_tree_amd import accept_walk
    tv = wl.tv
    n_req = len(ctxs)
    reqs = list(range(n_req))
    res_rng = np.random.default_rng(a.seed)

    def round_(n):
        per_req = trees[n]
        if n_req == 1 and a.residual > 0:   # verify, residual walk and commit in one call
            parents, tokens = per_req[0]
            path, _ = tv.residual_round(0, parents, tokens, a.residual, res_rng.random(32), logits=wl.logits)
            tv.set_history(0, hist[0], ctxs[0])
            return [len(path)]
        if n_req == 1:   # verify, accept walk and commit in one library call
            parents, tokens = per_req[0]
            _, _, path, _ = tv.round(0, parents, tokens, logits=wl.logits)
            tv.set_history(0, hist[0], ctxs[0])
            return [len(path)]
        am, _ = tv.verify_trees(reqs, [p for p, _ in per_req], [t for _, t in per_req], logits=wl.logits)
        lens = []
        for r in range(n_req):
            parents, tokens = per_req[r]
            path, _ = accept_walk(parents, tokens, am[r * n:(r + 1) * n])
            tv.commit(r, path)
            tv.set_history(r, hist[r], ctxs[r])
            lens.append(len(path))
        return lens

    for _ in range(a.warmup):
        for n in ns:
            round_(n)
    tv.profile_reset()
    tv.profile_enable(True, kern)
    per_n = {n: [] for n in ns}
    lens_seen = {n: [] for n in ns}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        for n in ns:
            s = time.perf_counter()
            lens = round_(n)
            per_n[n].append(time.perf_counter() - s)
            lens_seen[n].append(lens)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    k_ms, k_cnt = tv.profile_get(kern)
    tv.profile_enable(False)
    print(f"[bench] {shape.name} ctx {ctxs}: {a.steps} steps in {total:.3f} s", file=sys.stderr, flush=True)

    all_bytes = sum(model_bytes(shape, n, ctxs, lens, mods_on) for n in ns for lens in lens_seen[n])
    per = {}
    for n in ns:
        ms = float(np.median(per_n[n]) * 1e3)
        plen = [float(np.mean([l[r] for l in lens_seen[n]])) for r in range(n_req)]
        by = model_bytes(shape, n, ctxs, [int(round(x)) for x in plen], mods_on)
        key = str(n) if n_req == 1 else "+".join([str(n)] * n_req)
        per[key] = {"ms_median": round(ms, 4), "ms_min": round(float(np.min(per_n[n]) * 1e3), 4),
                    "GBps": round(by / ms / 1e6, 1), "frac_hbm": round(by / ms / 1e6 / HBM_PEAK_GBS, 4),
                    "rows_per_s": round(n * n_req / ms * 1e3, 1), "bytes": by,
                    "path_len": plen[0] if n_req == 1 else plen}
    ratio = per["16"]["ms_median"] / per["8"]["ms_median"] if "8" in per and "16" in per else None
    k_avg_ms = k_ms / max(k_cnt, 1)
    if kern == "gemm_head":
        kb = float(np.mean([head_bytes(shape, n * n_req) for n in ns]))
        kname = "gemm_head (k_gemm<EPI_HEAD>)"
        summary = "gemm_head_c1_layer_ctx1024_counters.md"
    else:
        kb = float(np.mean([gateup_bytes(shape, n * n_req) for n in ns]))
        kname = "gemm_gateup (k_gemm<EPI_SWIGLU>, split-K partials)"
        summary = "gemm_gateup_c2_stack64_ctx1024_counters.md"
    achieved = kb / (k_avg_ms * 1e-3) / 1e9
    counted = shape.name in ("c1_layer", "c2_stack64") and ctxs == [1024] and not mods_on
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic(summary) if counted else None,
            "kernel": kname, "avg_us": round(k_avg_ms * 1e3, 2), "bytes_per_launch": int(kb), "launches": k_cnt}
    return {"value": round(all_bytes / total / 1e9, 2), "ms_per_step": round(total / a.steps * 1e3, 4),
            "step_bytes": all_bytes // a.steps, "per_n": per,
            "ratio_16_over_8": round(ratio, 4) if ratio else None, "roofline": roof,
            "round_": round_}


def kernel_breakdown(tv, round_, ns):
    tv.profile_reset()
    tv.profile_enable(True, "")
    for _ in range(5):
        for n in ns:
            round_(n)
    kernels = {}
    for k in ("embed_norm", "resid_norm", "gemm_qkv", "rope_kv", "attn", "attn_combine", "gemm_o",
              "gemm_gateup", "splitk_finish", "gemm_down", "gemm_gate", "recur_tree", "gemm_head",
              "top2", "residual", "commit_kv", "commit_state"):
        ms, cnt = tv.profile_get(k)
        if cnt:
            kernels[k] = {"avg_us": round(ms / cnt * 1e3, 2), "launches": cnt}
    # prefix counts: "attn" also matches "attn_combine", "gemm_gate" also "gemm_gateup"
    for k, sub in (("attn", "attn_combine"), ("gemm_gate", "gemm_gateup")):
        if k in kernels and sub in kernels:
            ms, cnt = tv.profile_get(k)
            ms2, cnt2 = tv.profile_get(sub)
            if cnt > cnt2:
                kernels[k] = {"avg_us": round((ms - ms2) / (cnt - cnt2) * 1e3, 2), "launches": cnt - cnt2}
            else:
                del kernels[k]
    tv.profile_enable(False)
    return kernels


def describe(config, shape, ctxs, ns, a):
    wname = {"c1": "c1_layer: 1 x", "c2": "c2_stack64: 64 x",
             "c3": "c3_hybrid64: 48 recurrent + 16 attention layers x",
             "c3d": "c3d_delta64: 48 gated delta-rule + 16 attention layers x",
             "c4": "c4 on c2_stack64: 64 x"}[config]
    return (f"{wname} (hidden {shape.hidden}, {shape.n_qhead}q/{shape.n_kvhead}kv heads x {shape.head_dim}, "
            f"SwiGLU {shape.ffn}) + fp32 head V={shape.vocab}; KV cache {'/'.join(map(str, ctxs))} rows; "
            f"one step = verify+accept+commit of trees n={','.join(map(str, ns))}"
            + (" for 2 requests in one pass, modifiers on, wrong drafter" if config == "c4" else "")
            + (f"; sampled requests (temperature {a.temperature}, seed {a.seed})" if a.temperature > 0 else "")
            + (f"; residual tree sampling at temperature {a.residual}" if a.residual > 0 else ""))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(a verify does not shard: see the design notes on multi-GPU)", file=sys.stderr)
        sys.exit(2)
    import gc
    import torch
    import synth

    shape = {"c1": synth.C1, "c2": synth.C2, "c3": synth.C3, "c3d": synth.C3D, "c4": synth.C2}[a.config]
    ns = {"c1": NS, "c2": NS, "c3": (16,), "c3d": (16,), "c4": (16,)}[a.config]
    ctxs = [a.ctx, a.ctx2] if a.config == "c4" else [a.ctx]
    if a.lookup:
        return lookup_main(a)
    if a.prices:
        return prices_main(a, shape)
    if a.prefill:
        return prefill_main(a, shape)
    n_req = len(ctxs)
    mods_on = a.config == "c4"
    torch.cuda.init()
    if a.copy_probe:
        src_t = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst_t = torch.empty_like(src_t)
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t
    extra_ctx = [int(x) for x in a.extra_ctx.split(",") if x] if (a.config == "c2" and not a.no_extras) else []
    want_cpu = (not a.no_cpu_baseline and int(os.environ.get("RANK", "0")) == 0
                and a.config in ("c1", "c2"))
    wl = build_workload(a, shape, max(ctxs + extra_ctx) + 64, n_req, want_cpu)
    hist, kv, trees = setup(a, wl, shape, ns, ctxs, mods_on)
    kern = "gemm_head" if a.config == "c1" else "gemm_gateup"
    res = time_rounds(a, wl, shape, ns, ctxs, hist, trees, kern, mods_on)

    kernels = kernel_breakdown(wl.tv, res["round_"], ns) if a.kernel_breakdown else None
    cpu = None
    if want_cpu:
        cpu = cpu_baseline(shape, wl, kv, ctxs[0], {n: trees[n][0] for n in ns}, a.cpu_sample, ns)
        wl.host_weights = None
        gc.collect()

    out = {
        "metric": "ms per tree verify + achieved HBM GB/s at 8/16/24/32 nodes, 1k ctx, 1 GPU",
        "value": res["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(a.config, shape, ctxs, ns, a), "ctx": ctxs[0] if n_req == 1 else ctxs,
                   "tree_nodes": list(ns), "requests": n_req, "step_bytes": res["step_bytes"],
                   "sampling": {"temperature": a.temperature, "seed": a.seed} if a.temperature > 0 else None,
                   "residual_temperature": a.residual if a.residual > 0 else None},
        "per_n": res["per_n"],
        "ratio_16_over_8": res["ratio_16_over_8"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
    }
    # the same stack at the longer contexts (its own bytes: the caches read grow)
    for ctx in extra_ctx:
        h, _, tr = setup(a, wl, shape, ns, [ctx], False)
        r = time_rounds(a, wl, shape, ns, [ctx], h, tr, kern, False)
        out[f"ctx{ctx}"] = {"value": r["value"], "ms_per_step": r["ms_per_step"], "per_n": r["per_n"],
                            "ratio_16_over_8": r["ratio_16_over_8"],
                            "gateup_us": r["roofline"]["avg_us"], "gateup_frac": r["roofline"]["frac"]}
    if a.config == "c2" and not a.no_extras:
        # one layer + the head (the c1 workload): where the head's 1.56 GB dominates
        wl.tv.close()
        del wl
        gc.collect()
        torch.cuda.empty_cache()
        wl1 = build_workload(a, synth.C1, a.ctx + 64, 1, False)
        h, _, tr = setup(a, wl1, synth.C1, NS, [a.ctx], False)
        r = time_rounds(a, wl1, synth.C1, NS, [a.ctx], h, tr, "gemm_head", False)
        out["c1_layer"] = {"workload": describe("c1", synth.C1, [a.ctx], NS, a), "value": r["value"],
                           "ms_per_step": r["ms_per_step"], "per_n": r["per_n"],
                           "ratio_16_over_8": r["ratio_16_over_8"], "roofline": r["roofline"]}
        wl1.tv.close()
    if kernels:
        out["kernels"] = kernels
    print(json.dumps(out), flush=True)


def prefill_main(a, shape):
    """Dense prefill throughput: a prompt of --prefill uniform tokens through
    tv_prefill_dense in chunks of --chunk rows,
    with the dense gate/up GEMM's MFMA roofline and the chained (32-row)
    prefill timed once beside it."""
    import torch
    import synth
    import workloads
    n, chunk = a.prefill, a.chunk
    torch.cuda.init()
    print(f"[bench] building {shape.name} for a {n}-token prefill", file=sys.stderr, flush=True)
    wl = workloads.build(shape, max_ctx=n + 64, max_req=1, weight_device="cuda")
    tv = wl.tv
    prompt = synth.uniform_ids(n, shape.vocab, 5)

    def once():
        tv.set_history(0, [], 0)
        return tv.prefill_dense(0, prompt, chunk=chunk)

    for _ in range(a.warmup):
        once()
    print("[bench] warm", file=sys.stderr, flush=True)
    tv.profile_reset()
    tv.profile_enable(True, "pf_gemm_gateup")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        once()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    k_ms, k_cnt = tv.profile_get("pf_gemm_gateup")
    tv.profile_enable(False)
    kernels = None
    if a.kernel_breakdown:
        tv.profile_reset()
        tv.profile_enable(True, "")
        once()
        kernels = {}
        for k in ("pf_embed_norm", "pf_gemm_qkv", "pf_rope", "pf_attn_combine", "pf_gemm_o", "pf_norm",
                  "pf_gemm_gateup", "pf_gemm_down", "pf_gemm_gate", "pf_recur", "pf_commit_state",
                  "gemm_head", "top2"):
            ms, cnt = tv.profile_get(k)
            if cnt:
                kernels[k] = {"avg_us": round(ms / cnt * 1e3, 2), "launches": cnt}
        ms, cnt = tv.profile_get("pf_attn")
        ms2, cnt2 = tv.profile_get("pf_attn_combine")
        if cnt > cnt2:
            kernels["pf_attn"] = {"avg_us": round((ms - ms2) / (cnt - cnt2) * 1e3, 2), "launches": cnt - cnt2}
        tv.profile_enable(False)
    # the chained prefill (32-row verify passes, each committed) once, for comparison
    tv.set_history(0, [], 0)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tv.prefill(0, prompt)
    torch.cuda.synchronize()
    chain_s = time.perf_counter() - t1
    # gate/up: 2 * rows * (2 * ffn) * hidden flops per launch; launches cover every chunk of every layer
    chunks = []
    pos = 0
    while pos < n:
        k = min(n - pos, chunk - pos % chunk)
        chunks.append(k)
        pos += k
    flops = sum(2.0 * k * 2 * shape.ffn * shape.hidden for k in chunks) * len(shape.kinds)
    k_avg_ms = k_ms / max(k_cnt, 1)
    achieved = flops / len(chunks) / len(shape.kinds) / (k_avg_ms * 1e-3) / 1e12
    out = {
        "metric": "dense prefill tokens/s",
        "value": round(n * a.steps / total, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(total / a.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}: prefill of {n} uniform tokens in chunks of {chunk} rows",
                   "tokens": n, "chunk": chunk},
        "chained_prefill_tokens_per_s": round(n / chain_s, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 2500.0, 4), "traffic": None,
                     "kernel": "pf_gemm_gateup (SwiGLU: k_gemm_big when its tiles cover at least half the CUs, else k_gemm_dense<EPI_SWIGLU, 2>)", "avg_us": round(k_avg_ms * 1e3, 2),
                     "launches": k_cnt},
    }
    if kernels:
        out["kernels"] = kernels
    print(json.dumps(out), flush=True)


def prices_main(a, shape):
    """StairCut's verify price file for this workload on this GPU: median
    wall time of a verify (host call to host results) by context length,
    kind and rows, in the pages' stair-table format (one JSON line)."""
    import torch
    import workloads
    from greedy_draft_tree_amd.staircut import measure_prices
    lens = [int(x) for x in a.price_ctx.split(",")]
    torch.cuda.init()
    print(f"[bench] building {shape.name} for prices at {lens}", file=sys.stderr, flush=True)
    wl = workloads.build(shape, max_ctx=max(lens) + 64, max_req=1, weight_device="cuda")
    workloads.load_context(wl, 0, max(lens), seed=3, state_seed=6)
    t0 = time.perf_counter()
    table, steps = {}, []
    for L in lens:   # one length at a time, with progress
        part = measure_prices(wl.tv, 0, [L], reps=a.price_reps)
        table[str(L)] = part[str(L)]
        steps.append(part["step_ms"])
        print(f"[bench] prices at ctx {L} done ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    table["step_ms"] = float(np.median(steps))
    table["measured"] = (f"bench.py --prices --config {a.config}: median of {a.price_reps} verifies per count "
                         f"(host call to host results) on one MI355X, {time.strftime('%Y-%m-%d')}")
    table["workload"] = shape.name
    print(json.dumps(table), flush=True)


def lookup_main(a):
    """The lookup drafter's host cost per call (the pages give about 0.2 ms a
    lookup): the native tv_lookup_draft (orders 2..8, depth 31, 31 nodes) at
    each --price-ctx length on two texts, a quoting one (uniform ids that end
    by quoting 20 tokens of an earlier span: one vote, a 31-node chain) and a
    looping one (a 37-token cycle: a vote every cycle).  ``value`` is the
    quoting text at the longest length; ``cpu_baseline`` the oracle's plain
    Python on the same quoting texts."""
    import synth
    from greedy_draft_tree_amd.lookup import draft
    from oracle.lookup import lookup_draft as oracle_draft
    lens = [int(x) for x in a.price_ctx.split(",")]
    per, texts = {}, {}
    for L in lens:
        ids = synth.uniform_ids(L, 151936, 5)
        quote = np.concatenate([ids, ids[L // 3:L // 3 + 20]]).astype(np.int32)
        loop = np.asarray((list(range(37)) * (L // 37 + 2))[:L], np.int32)
        texts[L] = quote
        per[str(L)] = {}
        for name, text in (("quoting", quote), ("looping", loop)):
            draft(text)
            reps = max(20, 200 * 1024 // L)
            t0 = time.perf_counter()
            for _ in range(reps):
                t = draft(text)
            ms = (time.perf_counter() - t0) / reps * 1e3
            per[str(L)][name] = {"ms": round(ms, 4), "votes": t.votes, "nodes": len(t.parents),
                                 "match_order": t.match_order}
        print(f"[bench] lookup at ctx {L} done", file=sys.stderr, flush=True)
    cpu = None
    if not a.no_cpu_baseline:
        t0, calls = time.perf_counter(), 0
        while time.perf_counter() - t0 < 5.0 or calls < len(lens):
            oracle_draft(texts[lens[calls % len(lens)]].tolist())
            calls += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(dt / calls * 1e3, 3), "unit": "ms per call", "cores": 1, "kind": "oracle",
               "sample": f"{calls} calls over the quoting texts at {lens} (plain Python, one thread)"}
    L = str(max(lens))
    print(json.dumps({"metric": "lookup drafter ms per call (host)", "value": per[L]["quoting"]["ms"],
                      "unit": "ms", "n_gpus": 0, "higher_is_better": False, "vs_baseline": None,
                      "dtype": "int32", "data": "synthetic",
                      "config": {"workload": f"lookup drafter, orders 2..8, depth 31, 31 nodes, text of {L} ids"},
                      "per_ctx": per, "cpu_baseline": cpu}), flush=True)


def cpu_baseline(shape, wl, kv, ctx, trees, sample, ns):
    """The CPU oracle (brute-force tree scorer) on the same trees."""
    import oracle
    w_cpu = wl.host_weights
    kv_cpu = {k: v[:, :ctx].cpu() for k, v in kv.items()}
    orc = oracle.Oracle(shape, w_cpu)
    seq = orc.new_seq(cap=ctx + 40, kv=kv_cpu, ctx_len=ctx)
    ns = ns if sample == "full" else (8,)
    t0 = time.perf_counter()
    by, trees_done, passes = 0, 0, 0
    while True:   # whole passes over the sample until at least MIN_CPU_S seconds
        for n in ns:
            parents, tokens = trees[n]
            orc.tree_scores(seq, parents, tokens)
            by += model_bytes(shape, n, [ctx], [1])
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
