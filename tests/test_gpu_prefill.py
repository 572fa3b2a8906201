"""GPU parity of the prefill path against the oracle.

Part 2, "PCP: split tokens, not heads": the indexer scores every earlier token of every prompt
token.  Part 2, "Try it": prompts within the 2,048-token top-K stay on the sparse-MLA (MQA)
kernel.  The prefill of P new tokens at the end of an L-token context is the oracle's step
with S = P queries (query i sees the rows t < L - P + 1 + i): the GPU top-K of each query must
match the oracle's within the tie band, and the attention over that (checked) selection must
match the oracle's dense softmax over the same rows.  At 32K tokens the oracle checks sampled queries one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from hs_harness import GpuWorkload, check_attention, check_topk

pytestmark = pytest.mark.gpu


def _prefill(gw: GpuWorkload, b: int, P: int, with_topk: bool = True, attend_last: int | None = None):
    """Prefill of request b's last P tokens: the indexer over all P (unless with_topk is False),
    attention for the last `attend_last` of them (all by default), on the GPU's selection."""
    wl = gw.wl
    L = int(wl.ctx[b])
    A = P if attend_last is None else attend_last
    qidx = synth.prefill_qidx(wl, b, P)
    w = synth.prefill_head_weights(wl, b, P)
    q = synth.prefill_mla_q_range(wl, b, P - A, A)       # token i's draw does not depend on P
    topk = None
    if with_topk:
        topk = torch.empty((P, wl.topk), dtype=torch.int32, device=gw.dev)
        gw.ctx.prefill_index_topk(b, gw.to_dev(qidx), torch.from_numpy(w).to(gw.dev), L, topk)
    out = torch.empty((A, 64, 512), dtype=torch.bfloat16, device=gw.dev)
    lse = torch.empty((A, 64), dtype=torch.float32, device=gw.dev)
    # the last A tokens of the prefill are a prefill of A tokens of the same context
    gw.ctx.prefill(0, b, gw.to_dev(q), topk[P - A:] if topk is not None else None, L, gw.sm_scale,
                   out, lse)
    torch.cuda.synchronize()
    return qidx, w, q, topk, out, lse


def _check_queries(gw, b, P, qidx, w, q, topk, out, lse, queries, attend_last=None):
    """Query i (of the P): its top-K against the oracle's scores (tie band), and, if it is one of
    the last `attend_last`, its attention over the GPU's selection against the oracle."""
    wl = gw.wl
    L = int(wl.ctx[b])
    A = P if attend_last is None else attend_last
    keys = gw.keys(b)[:L]
    tk = topk.cpu().numpy() if topk is not None else None
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    for i in queries:
        visible = L - P + 1 + i
        if tk is not None:
            sc = oracle.indexer_scores(qidx[i:i + 1], w[i:i + 1], keys[:visible])[0]
            check_topk(tk[i], sc, wl.topk)
            toks = tk[i][tk[i] >= 0]
        else:
            toks = np.arange(visible)
        a = i - (P - A)
        if a < 0:
            continue
        rows = synth.latent_tokens(wl, b, 0, toks)
        o_ref, l_ref = oracle.attention(q[a], oracle.decode_latent_rows(rows, wl.kv_dtype), gw.sm_scale)
        check_attention(o[a], l[a], o_ref, l_ref)


def test_prefill_chunk_toy():
    # request 1 prefills its last 301 tokens (L = 1333): chunks of 2 x 4 queries, the last chunk
    # holding one full group of 4 and a group of 1; K = 128 < L, so the indexer selects
    wl = synth.toy(seed=41, batch=2, queries=4, ctx=(700, 1333), topk=128, steps=1,
                   residency=[(synth.RES_FULL, 1.0)] * 2)
    gw = GpuWorkload(wl)
    print("[prefill] toy 301 of 1333", flush=True)
    P = 301
    qidx, w, q, topk, out, lse = _prefill(gw, 1, P)
    _check_queries(gw, 1, P, qidx, w, q, topk, out, lse, range(P))
    assert gw.ctx.device_error() == 0
    gw.close()


def test_force_mqa_prompt_within_topk():
    # a whole 700-token prompt with K = 1024: every token attends to every row it sees, on the
    # sparse kernel; with and without the indexer's (select-all) top-K the result is bitwise equal
    wl = synth.toy(seed=42, batch=1, queries=3, ctx=(700,), topk=1024, steps=1,
                   residency=[(synth.RES_FULL, 1.0)])
    gw = GpuWorkload(wl, max_batch=8)
    print("[prefill] force-MQA 700", flush=True)
    P = 700
    qidx, w, q, topk, out, lse = _prefill(gw, 0, P)
    tk = topk.cpu().numpy()
    for i in range(P):
        assert np.array_equal(tk[i, :i + 1], np.arange(i + 1)) and (tk[i, i + 1:] == -1).all()
    _, _, _, _, out2, lse2 = _prefill(gw, 0, P, with_topk=False)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    _check_queries(gw, 0, P, qidx, w, q, None, out2, lse2, range(0, P, 7))
    assert gw.ctx.device_error() == 0
    gw.close()


def test_prefill_32k_sampled():
    # a 32,768-token prompt, K = 2,048: sampled queries (the first, those around K, the last)
    # checked one by one against the oracle
    wl = synth.toy(seed=43, batch=1, queries=4, ctx=(32768,), topk=2048, steps=1,
                   residency=[(synth.RES_FULL, 1.0)])
    gw = GpuWorkload(wl, max_batch=64)
    print("[prefill] 32K", flush=True)
    P, A = 32768, 2048
    qidx, w, q, topk, out, lse = _prefill(gw, 0, P, attend_last=A)
    sample = [0, 1, 2046, 2047, 2048, 2049, 4095, 9000, 16383, 20001, 30719, 30720, 31500, 32766, 32767]
    _check_queries(gw, 0, P, qidx, w, q, topk, out, lse, sample, attend_last=A)
    assert gw.ctx.device_error() == 0
    gw.close()


def test_prefill_argument_errors():
    import sparse_mla_attention_score_amd.hisparse as hsb
    wl = synth.toy(seed=44, batch=1, queries=1, ctx=(3000,), topk=256, steps=1,
                   residency=[(synth.RES_FULL, 1.0)])
    gw = GpuWorkload(wl)
    q = torch.zeros((4, 64, 576), dtype=torch.bfloat16, device=gw.dev)
    out = torch.empty((4, 64, 512), dtype=torch.bfloat16, device=gw.dev)
    with pytest.raises(hsb.HiSparseError):       # L > K needs a top-K
        gw.ctx.prefill(0, 0, q, None, 3000, gw.sm_scale, out)
    with pytest.raises(hsb.HiSparseError):       # P > L
        gw.ctx.prefill(0, 0, q, None, 3, gw.sm_scale, out)
    with pytest.raises(hsb.HiSparseError):       # request outside max_batch
        gw.ctx.prefill(0, 1, q, None, 200, gw.sm_scale, out)
    assert gw.ctx.device_error() == 0
    gw.close()
