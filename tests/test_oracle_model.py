"""Pins of the oracle's model forward and tree scorer.

* With every rounding point off, the oracle's one-token steps equal an
  independent library implementation of the same decoder (transformers'
  Llama in fp64, a causal forward over the whole sequence) -- this catches a
  dropped term, a wrong sign or index, a transposed operand or a misplaced
  norm weight anywhere in the forward.
* The tree scorer's row i equals sequential decoding of node i's ancestor
  prefix ("Drafters and tree verify", The round, step 2;
  "Algorithm and correctness contract", Target position and batching), both
  bitwise within the oracle and against the library's causal forward.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore")

SHAPE = synth.C0


def _weights(seed=0, random_norms=True):
    w = synth.weights(SHAPE, seed=seed)
    if random_norms:
        g = torch.Generator().manual_seed(99 + seed)
        for k in list(w):
            if k.endswith("norm"):
                w[k] = (1.0 + 0.3 * torch.randn(w[k].shape, generator=g)).to(torch.bfloat16)
    return w


def _hf_model(w):
    from transformers import LlamaConfig, LlamaForCausalLM
    s = SHAPE
    cfg = LlamaConfig(vocab_size=s.vocab, hidden_size=s.hidden, intermediate_size=s.ffn,
                      num_hidden_layers=s.n_layer, num_attention_heads=s.n_qhead,
                      num_key_value_heads=s.n_kvhead, head_dim=s.head_dim,
                      rms_norm_eps=s.eps, rope_theta=s.rope_theta, tie_word_embeddings=False,
                      attention_bias=False, mlp_bias=False, max_position_embeddings=4096,
                      attn_implementation="eager")
    m = LlamaForCausalLM(cfg).double().eval()
    QD, KD = s.n_qhead * s.head_dim, s.n_kvhead * s.head_dim
    sd = {"model.embed_tokens.weight": w["emb"], "model.norm.weight": w["final_norm"],
          "lm_head.weight": w["head"]}
    for l in range(s.n_layer):
        p, q = f"layers.{l}.", f"model.layers.{l}."
        wqkv = w[p + "wqkv"]
        sd[q + "self_attn.q_proj.weight"] = wqkv[:QD]
        sd[q + "self_attn.k_proj.weight"] = wqkv[QD:QD + KD]
        sd[q + "self_attn.v_proj.weight"] = wqkv[QD + KD:]
        sd[q + "self_attn.o_proj.weight"] = w[p + "wo"]
        sd[q + "mlp.gate_proj.weight"] = w[p + "wg"]
        sd[q + "mlp.up_proj.weight"] = w[p + "wu"]
        sd[q + "mlp.down_proj.weight"] = w[p + "wd"]
        sd[q + "input_layernorm.weight"] = w[p + "attn_norm"]
        sd[q + "post_attention_layernorm.weight"] = w[p + "ffn_norm"]
    sd = {k: v.to(torch.float64) for k, v in sd.items()}
    missing, unexpected = m.load_state_dict(sd, strict=False)
    assert not unexpected, unexpected
    assert all("rotary" in k for k in missing), missing
    # exact fp64 RoPE frequencies (the library computes them in fp32)
    D = s.head_dim
    exact = s.rope_theta ** (-(2.0 * torch.arange(D // 2, dtype=torch.float64)) / D)
    for mod in m.modules():
        if hasattr(mod, "inv_freq"):
            mod.inv_freq = exact.clone()
            if hasattr(mod, "original_inv_freq"):
                mod.original_inv_freq = exact.clone()
    return m


# The library keeps its RMSNorm, softmax and RoPE tables in fp32 even in an
# fp64 model, so agreement is at fp32 level; any structural mistake is O(1).
TOL = 3e-6


def _hf_logits(m, ids):
    with torch.no_grad():
        return m(torch.tensor([list(ids)], dtype=torch.long)).logits[0].numpy()


@pytest.fixture(scope="module")
def pair():
    w = _weights()
    return oracle.Oracle(SHAPE, w, exact=True), _hf_model(w), w


def test_exact_forward_matches_library_llama(pair):
    orc, hf, _ = pair
    ids = synth.uniform_ids(24, SHAPE.vocab, 11)
    seq = orc.new_seq(cap=64)
    got = np.stack([seq.step(int(t)) for t in ids])
    want = _hf_logits(hf, ids)
    scale = np.abs(want).max()
    np.testing.assert_allclose(got, want, rtol=0, atol=TOL * scale)


def test_exact_tree_rows_match_library_prefix_decode(pair):
    orc, hf, _ = pair
    prompt = synth.uniform_ids(9, SHAPE.vocab, 12)
    seq = orc.new_seq(cap=64)
    seq.commit(prompt)
    parents = synth.random_tree(11, 5)
    tokens = synth.tree_tokens(parents, SHAPE.vocab, 6, root_token=int(prompt[-1] + 1) % SHAPE.vocab)
    rows = orc.tree_scores(seq, parents, tokens)
    for i in range(len(parents)):
        ctx = list(prompt) + oracle.path_tokens(parents, tokens, i)
        want = _hf_logits(hf, ctx)[-1]
        np.testing.assert_allclose(rows[i], want, rtol=0, atol=TOL * np.abs(want).max())


@pytest.fixture(scope="module")
def rounded():
    w = synth.weights(SHAPE, seed=0)
    return oracle.Oracle(SHAPE, w, exact=False)


def test_rounded_tree_rows_equal_sequential_decode(rounded):
    orc = rounded
    prompt = synth.uniform_ids(17, SHAPE.vocab, 1)
    base = orc.new_seq(cap=64)
    base.commit(prompt)
    for seed, parents in [(2, synth.c0_tree()), (3, synth.spine_tree(16, 3)),
                          (4, synth.chain_tree(6)), (5, synth.bush_tree(5))]:
        tokens = synth.tree_tokens(parents, SHAPE.vocab, seed, root_token=7)
        rows = orc.tree_scores(base, parents, tokens)
        for i in range(len(parents)):
            s = orc.new_seq(cap=64)
            s.commit(prompt)
            last = s.commit(oracle.path_tokens(parents, tokens, i))
            np.testing.assert_array_equal(rows[i], last)


def test_rounded_values_sit_on_their_grids(rounded):
    orc = rounded
    seq = orc.new_seq(cap=16)
    logits = seq.commit(synth.uniform_ids(5, SHAPE.vocab, 2))
    # KV rows are bf16 values, logits fp32 values
    for l in seq.K:
        k = seq.K[l][:, :5]
        v = seq.V[l][:, :5]
        np.testing.assert_array_equal(oracle.bf16_round(k), k)
        np.testing.assert_array_equal(oracle.bf16_round(v), v)
    np.testing.assert_array_equal(oracle.f32(logits), logits)


def test_rounded_close_to_exact(rounded):
    # bf16 rounding points move the logits by a small amount only
    w = synth.weights(SHAPE, seed=0)
    ex = oracle.Oracle(SHAPE, w, exact=True)
    ids = synth.uniform_ids(12, SHAPE.vocab, 4)
    a, b = rounded.new_seq(cap=16), ex.new_seq(cap=16)
    la = np.stack([a.step(int(t)) for t in ids])
    lb = np.stack([b.step(int(t)) for t in ids])
    err = np.abs(la - lb).max()
    assert 0 < err < 0.05 * np.abs(lb).std()


def test_rope_position_zero_is_identity_and_relative(rounded):
    orc = oracle.Oracle(SHAPE, synth.weights(SHAPE, seed=0), exact=True)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((3, SHAPE.head_dim))
    k = rng.standard_normal((3, SHAPE.head_dim))
    np.testing.assert_array_equal(orc.rope(q, 0), q)
    d1 = np.sum(orc.rope(q, 10) * orc.rope(k, 3), axis=1)
    d2 = np.sum(orc.rope(q, 107) * orc.rope(k, 100), axis=1)
    np.testing.assert_allclose(d1, d2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(orc.rope(q, 55), axis=1), np.linalg.norm(q, axis=1))


def test_exact_tree_over_synthetic_cache_matches_library(pair):
    # Rows [0, ctx) of every layer's cache are given (already rotated); the
    # tree's root sits at position ctx.  The library takes the same rows as
    # a pre-filled cache.
    from transformers import DynamicCache
    orc, hf, _ = pair
    ctx = 37
    kv = synth.kv_cache(SHAPE, ctx, seed=3, cap=64)
    seq = orc.new_seq(cap=64, kv=kv, ctx_len=ctx)
    parents = synth.spine_tree(9, 2)
    tokens = synth.tree_tokens(parents, SHAPE.vocab, 8, root_token=5)
    rows = orc.tree_scores(seq, parents, tokens)
    for i in (0, 3, len(parents) - 1):
        cache = DynamicCache()
        for l in range(SHAPE.n_layer):
            cache.update(kv[(l, "k")][None, :, :ctx].to(torch.float64),
                         kv[(l, "v")][None, :, :ctx].to(torch.float64), l)
        ids = oracle.path_tokens(parents, tokens, i)
        pos = torch.arange(ctx, ctx + len(ids))[None]
        with torch.no_grad():
            want = hf(torch.tensor([ids]), past_key_values=cache, position_ids=pos,
                      use_cache=True).logits[0, -1].numpy()
        np.testing.assert_allclose(rows[i], want, rtol=0, atol=TOL * np.abs(want).max())
