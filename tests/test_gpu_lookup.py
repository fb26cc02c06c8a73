"""The lookup drafter in the verify loop on the GPU (MI355X only).

"Drafters and tree verify", The lookup drafter; "Exactness", The promise: a
drafter changes how fast the text arrives, not what it says.  Each round
drafts from the request's own text (prompt and output so far) with
tv_lookup_draft, verifies the tree, walks it and commits; every row is held
to the oracle (logits within tolerance, argmax equal unless the oracle's gap
is at most one bf16 ulp), so the emitted text is the model's greedy text.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def test_c0_lookup_drafter_rounds():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import workloads
    from test_gpu_parity import check_rows
    from greedy_draft_tree_amd.lookup import draft
    wl = workloads.build(synth.C0, max_ctx=1024, max_req=1, weight_device="cuda", host_copy=True)
    orc = oracle.Oracle(synth.C0, wl.host_weights)
    base = synth.uniform_ids(80, synth.C0.vocab, 21)
    prompt = np.concatenate([base, base[10:50]])   # ends by quoting an earlier span
    wl.tv.set_history(0, [], 0)
    wl.tv.prefill(0, prompt[:-1])
    seq = orc.new_seq(cap=1024)
    seq.commit(prompt[:-1])
    text = [int(t) for t in prompt]
    fired, emitted_total = 0, 0
    for r in range(24):
        t = draft(text, 2, 8, 31, 31)
        parents, tokens = t.parents, t.tokens
        fired += len(parents) > 1
        print(f"[case] lookup round {r}: {len(parents)} rows, order {t.match_order}, {t.votes} votes", flush=True)
        am, gap = wl.tv.verify_tree(0, parents, tokens, logits=wl.logits)
        ol = orc.tree_scores(seq, parents, tokens)
        check_rows(wl.logits[:len(parents)].cpu().numpy(), am, gap, ol, parents, tokens, seq.history,
                   what=f"lookup round {r}")
        path, emitted = oracle.accept_walk(parents, tokens, am)
        wl.tv.commit(0, path)
        seq.commit([int(tokens[i]) for i in path])
        assert wl.tv.ctx_len(0) == seq.ctx_len
        text += [int(x) for x in emitted]
        emitted_total += len(emitted)
    print(f"[case] lookup: {emitted_total} tokens in 24 rounds, the drafter fired in {fired}", flush=True)
    assert fired > 0 and emitted_total >= 24
