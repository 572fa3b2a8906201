"""Pins of the oracle as the prefill path uses it.

Part 2, "PCP: split tokens, not heads": the indexer scores every earlier token of every prompt
token, a cost quadratic in the prompt length.  Part 2, "Try it": with sparse_mla_force_mqa,
prompts within the 2,048-token top-K stay on the sparse-MLA (MQA) kernel instead of dense
MHA, so every KV row serves all heads.

The prefill of P new tokens at the end of an L-token context is the oracle's step with S = P
queries: query i sees the rows t < L - P + 1 + i.
"""
import numpy as np
import torch

import oracle


def _bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_prefill_indexer_is_causal_brute_force():
    rng = np.random.default_rng(40)
    L, P = 37, 9
    q = _bf16_bits(rng, (P, 32, 128))
    w = rng.uniform(0, 1, (P, 32)).astype(np.float32)
    keys = rng.standard_normal((L, 128))
    got = oracle.indexer_scores(q, w, keys)
    qf = oracle.bf16_decode(q).reshape(P, 32, 128)
    for i in range(P):
        visible = L - P + 1 + i
        assert got[i].shape == (visible,)
        for t in range(visible):
            s = 0.0
            for h in range(32):
                d = sum(float(qf[i, h, k]) * float(keys[t, k]) for k in range(128))
                s += float(w[i, h]) * max(d, 0.0)
            assert abs(got[i][t] - s) <= 1e-9 * max(1.0, abs(s))


def test_force_mqa_prefill_equals_causal_sdpa():
    # a prompt shorter than top-K selects every earlier row: the sparse kernel's answer is dense
    # causal attention with one KV head broadcast to all 64 query heads
    rng = np.random.default_rng(41)
    L, P, K = 50, 20, 2048
    q = _bf16_bits(rng, (P, 64, 576))
    latent = rng.standard_normal((L, 576))
    scale = 1.0 / np.sqrt(576.0)
    outs, lses = [], []
    for i in range(P):
        visible = L - P + 1 + i
        tk = oracle.topk_select(np.zeros(visible), K)
        rows = tk[tk >= 0]
        assert np.array_equal(rows, np.arange(visible))
        o, l = oracle.attention(q[i], latent[rows], scale)
        outs.append(o)
        lses.append(l)
    qt = torch.from_numpy(oracle.bf16_decode(q).reshape(P, 64, 576)).permute(1, 0, 2)   # [64][P][576]
    k = torch.from_numpy(latent)[None].expand(64, L, 576)
    v = torch.from_numpy(latent[:, :512])[None].expand(64, L, 512)
    mask = torch.zeros(P, L, dtype=torch.bool)
    for i in range(P):
        mask[i, :L - P + 1 + i] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=scale)
    ref = ref.permute(1, 0, 2).numpy()                                                    # [P][64][512]
    assert np.allclose(np.stack(outs), ref, rtol=1e-10, atol=1e-12)
    logits = np.einsum("phd,ld->phl", oracle.bf16_decode(q).reshape(P, 64, 576), latent) * scale
    for i in range(P):
        lv = logits[i, :, :L - P + 1 + i]
        m = lv.max(axis=1)
        assert np.allclose(lses[i], m + np.log(np.exp(lv - m[:, None]).sum(axis=1)), rtol=1e-12)


def test_prefill_query_equals_single_decode_query():
    # query i of a prefill is the single decode query of a context that ends at its own row
    rng = np.random.default_rng(42)
    L, P = 300, 40
    q = _bf16_bits(rng, (P, 32, 128))
    w = rng.uniform(0, 1, (P, 32)).astype(np.float32)
    keys = rng.standard_normal((L, 128))
    full = oracle.indexer_scores(q, w, keys)
    for i in (0, 7, 39):
        one = oracle.indexer_scores(q[i:i + 1], w[i:i + 1], keys[:L - P + 1 + i])[0]
        assert np.array_equal(full[i], one)
        assert np.array_equal(oracle.topk_select(full[i], 64), oracle.topk_select(one, 64))
