"""GPU parity of the three C ABI calls against the CPU oracle on seeded synthetic workloads.

Stage-isolated: the top-K is checked against the oracle's scores; the resolver is fed the
oracle's top-K and must reproduce row ids, stats and hot-buffer state bit for bit; the decode
runs on those row ids and is checked against the oracle's dense softmax over the oracle's
selection.  Content: every resolved row holds its token's canonical bytes in every layer.
"""
import numpy as np
import pytest
import torch

import synth
from hs_harness import GpuWorkload, check_attention, check_content, check_topk

pytestmark = pytest.mark.gpu


def run_isolated(gw: GpuWorkload, steps: int, layers=None, label=""):
    wl = gw.wl
    B, S, K = wl.batch, wl.queries, wl.topk
    layers = range(wl.n_layers) if layers is None else layers
    worst = 0.0
    for step in range(steps):
        print(f"[{label or wl.name}] step {step}", flush=True)
        qidx, q, ctx_lens = gw.inputs(step)
        tk_gpu = gw.gpu_topk(qidx, ctx_lens).cpu().numpy()
        tk_ref = np.empty_like(tk_gpu)
        for b in range(B):
            ref, sc = gw.oracle_topk(b, qidx, int(ctx_lens[b]))
            tk_ref[b] = ref
            for j in range(S):
                check_topk(tk_gpu[b, j], sc[j], K)
        rows_dev, stats_dev = gw.gpu_resolve(torch.from_numpy(tk_ref).to(gw.dev), ctx_lens)
        rows, stats = rows_dev.cpu().numpy(), stats_dev.cpu().numpy()
        for b in range(B):
            rows_ref, _, st_ref = gw.oracle_resolve(b, tk_ref[b])
            assert np.array_equal(rows[b], rows_ref), f"row ids differ, request {b} step {step}"
            assert tuple(int(x) for x in stats[b]) == st_ref, f"stats {stats[b]} vs {st_ref}"
        st_tok, st_stamp, t2s, req_step = gw.ctx.hot_state()
        for b in range(B):
            o = gw.states[b]
            assert np.array_equal(st_tok[b], o.slot_token), f"slot_token request {b}"
            assert np.array_equal(st_stamp[b], o.slot_stamp), f"slot_stamp request {b}"
            assert np.array_equal(t2s[b], o.tok2slot), f"tok2slot request {b}"
            assert req_step[b] == step + 1
        for b in range(B):
            check_content(gw, b, rows[b].ravel(), tk_ref[b].ravel())
        for layer in layers:
            out, lse = gw.gpu_decode(layer, q, rows_dev, ctx_lens)
            out = out.float().cpu().numpy().astype(np.float64)
            lse = lse.cpu().numpy().astype(np.float64)
            for b in range(B):
                for j in range(S):
                    toks = tk_ref[b, j][tk_ref[b, j] >= 0]
                    o_ref, l_ref = gw.oracle_attention(b, j, layer, toks, q)
                    worst = max(worst, check_attention(out[b, j], lse[b, j], o_ref, l_ref))
        assert gw.ctx.device_error() == 0
    print(f"[{label or wl.name}] worst relative L2 {worst:.2e}", flush=True)


def test_toy_fp8_single_query():
    gw = GpuWorkload(synth.toy(seed=1, batch=2, queries=1, ctx=(700, 1333), topk=16, steps=4))
    run_isolated(gw, 4)
    gw.close()


def test_toy_fp8_mtp_union_resolve():
    wl = synth.toy(seed=2, batch=3, queries=4, ctx=(700, 1333, 97), topk=16, steps=4)
    gw = GpuWorkload(wl)
    run_isolated(gw, 4)
    gw.close()


def test_toy_bf16_rows_and_keys():
    wl = synth.toy(seed=3, batch=2, queries=2, ctx=(2000, 4097), topk=64, kv_dtype=0, idx_dtype=0,
                   steps=3)
    gw = GpuWorkload(wl)
    run_isolated(gw, 3)
    gw.close()


def test_toy_indexshare_four_layers_mixed_residency():
    wl = synth.toy(seed=4, batch=3, queries=1, ctx=(3000, 5000, 1500), topk=64, n_layers=4,
                   residency=[(synth.RES_FULL, 1.0), (synth.RES_HYBRID, 0.25), (synth.RES_PREFIX, 0.0)],
                   steps=3)
    gw = GpuWorkload(wl)
    run_isolated(gw, 3)
    gw.close()


@pytest.mark.parametrize("queries,idx_dtype", [(3, 1), (3, 0), (4, 0)],
                         ids=["s3_fp8_keys", "s3_bf16_keys", "s4_bf16_keys"])
def test_lists_and_scores_in_one_call(queries, idx_dtype):
    # S = 3: one pair of queries and a lone third share each tile (a score store and a list
    # store per pair and per lone query); FP8 key tiles go through the LDS ring, bf16 keys
    # through registers.  Step 0 selects from the scores, later steps from the candidate lists;
    # the 2,000-token request leaves no margin for a guess and is selected from its scores in
    # every step.
    wl = synth.toy(seed=12, batch=3, queries=queries, ctx=(5000, 2000, 9000), topk=256, steps=4,
                   idx_dtype=idx_dtype)
    gw = GpuWorkload(wl)
    run_isolated(gw, 4)
    from_list, from_scores = gw.ctx.select_paths()
    print(f"selections from the candidate list {from_list}, from all scores {from_scores}")
    assert from_list + from_scores == 4 * wl.batch * wl.queries
    assert from_scores >= 4 * wl.queries  # request 1 in every call, and the first call
    assert from_list >= 2 * 2 * wl.queries  # requests 0 and 2 from the second call on
    gw.close()


def test_topk2048_ragged_and_short_contexts():
    # several 64-row tiles, a ragged tail, and one context shorter than K (selects everything)
    wl = synth.toy(seed=5, batch=3, queries=1, ctx=(10000, 1500, 6100), topk=2048, steps=2)
    gw = GpuWorkload(wl)
    run_isolated(gw, 2)
    gw.close()


def test_minimum_and_page_boundary_contexts():
    # MTP3 over a context of exactly S tokens (the first query sees a single token, so its
    # top-K is one token and 15 padding entries), contexts that end on a page boundary (64, 128)
    # and one with a single token on its second page (65); each grows by S per step
    wl = synth.toy(seed=9, batch=4, queries=4, ctx=(4, 64, 65, 128), topk=16, steps=3)
    gw = GpuWorkload(wl)
    run_isolated(gw, 3)
    gw.close()


def test_select_multipass_path():
    # a one-entry on-chip candidate cap forces the general radix path of the select
    wl = synth.toy(seed=6, batch=2, queries=2, ctx=(5000, 2600), topk=256, steps=2)
    gw = GpuWorkload(wl, topk_lds_candidates=1)
    run_isolated(gw, 2)
    gw.close()


def test_select_from_candidate_list():
    # From the second call on, the sweep lists the tokens above each query's guess and the
    # select works from that list whenever the histogram proves it complete; every call's
    # top-K is still checked against the oracle.  The first call has no guess.
    wl = synth.toy(seed=7, batch=3, queries=2, ctx=(9000, 6000, 12000), topk=256, steps=5)
    gw = GpuWorkload(wl)
    run_isolated(gw, 5)
    from_list, from_scores = gw.ctx.select_paths()
    per_call = wl.batch * wl.queries
    print(f"selections from the candidate list {from_list}, from all scores {from_scores}")
    assert from_list + from_scores == 5 * per_call
    assert from_scores >= per_call  # the first call reads every score
    assert from_list >= 3 * per_call
    gw.close()


def test_select_falls_back_when_the_guess_misses():
    # The head weights are scaled by a power of two between calls.  The top-K is unchanged in
    # exact arithmetic, but every score moves by that factor, so the guess the previous call
    # left is too high (x0.25: too few tokens are listed) or far too low (x4 after x0.25: the
    # list's segments overflow).  The select must then read every score, and still match the
    # oracle; the call after each miss uses the list again.
    wl = synth.toy(seed=8, batch=2, queries=2, ctx=(9000, 12000), topk=256, steps=5)
    gw = GpuWorkload(wl)
    base = gw.w_np.copy()
    factors = [1.0, 0.25, 0.25, 4.0, 4.0]
    for step, f in enumerate(factors):
        gw.w_np = base * f
        gw.w = torch.from_numpy(gw.w_np).to(gw.dev)
        qidx, _, ctx_lens = gw.inputs(step)
        print(f"[guess misses] step {step} weights x{f}", flush=True)
        tk = gw.gpu_topk(qidx, ctx_lens).cpu().numpy()
        for b in range(wl.batch):
            _, sc = gw.oracle_topk(b, qidx, int(ctx_lens[b]))
            for j in range(wl.queries):
                check_topk(tk[b, j], sc[j], wl.topk)
    from_list, from_scores = gw.ctx.select_paths()
    per_call = wl.batch * wl.queries
    print(f"selections from the candidate list {from_list}, from all scores {from_scores}")
    assert from_list + from_scores == len(factors) * per_call
    assert from_scores >= 3 * per_call  # the first call and the two misses
    assert from_list >= per_call
    assert gw.ctx.device_error() == 0
    gw.close()


def test_select_rescores_only_the_queries_whose_list_misses():
    # At step 2 only request 1's head weights drop by x0.25, so only its two queries' lists
    # fall short of K: they are flagged, rescored (the rescoring sweep skips the other
    # requests) and selected from their scores, while the other requests' queries are served
    # by their lists in the same call.  Every call's top-K is checked against the oracle.
    wl = synth.toy(seed=11, batch=3, queries=2, ctx=(9000, 12000, 7000), topk=256, steps=4)
    gw = GpuWorkload(wl)
    base = gw.w_np.copy()
    paths = []
    for step in range(4):
        w = base.copy()
        if step >= 2:
            w[1] *= 0.25
        gw.w_np = w
        gw.w = torch.from_numpy(w).to(gw.dev)
        qidx, _, ctx_lens = gw.inputs(step)
        print(f"[partial rescore] step {step}", flush=True)
        tk = gw.gpu_topk(qidx, ctx_lens).cpu().numpy()
        for b in range(wl.batch):
            _, sc = gw.oracle_topk(b, qidx, int(ctx_lens[b]))
            for j in range(wl.queries):
                check_topk(tk[b, j], sc[j], wl.topk)
        paths.append(gw.ctx.select_paths())
    per_call = wl.batch * wl.queries
    from_list = [paths[i][0] - (paths[i - 1][0] if i else 0) for i in range(4)]
    from_scores = [paths[i][1] - (paths[i - 1][1] if i else 0) for i in range(4)]
    print(f"per call: from the list {from_list}, from the scores {from_scores}")
    assert all(from_list[i] + from_scores[i] == per_call for i in range(4))
    assert from_scores[0] == per_call  # no guesses yet
    # request 1's two queries from their scores, the other requests' from their lists
    assert from_scores[2] >= 2 and from_list[2] >= per_call - 3
    assert from_list[3] >= per_call - 1  # request 1 has a guess again
    assert gw.ctx.device_error() == 0
    gw.close()


@pytest.mark.parametrize("queries,ctx", [(4, (300000, 600000)), (2, (200000, 300000))],
                         ids=["s4_300k_600k", "s2_200k_300k"])
def test_resolver_union_paths_long_contexts(queries, ctx):
    # The resolver builds a request's union of its S lists through a token bitmap: with the
    # bitmap in one LDS array (contexts up to 32 tokens per union slot) each entry's place in the
    # union is read off the bitmap; with a longer context the bitmap spans two LDS arrays (up to
    # 64 tokens per slot), and beyond that it lives in workspace memory, and the places are found
    # by binary search.  K = 2,048 gives 8,192 slots at S = 4 and 4,096 at S = 2, so each
    # request here takes one of the two longer paths.  The lists are synthetic: each step draws
    # 2,600 tokens per request, keeping 80 % of the last step's, and each query takes 2,048 of
    # them, so the queries share most tokens and the hot buffer sees hits, misses and evictions.
    S, K = queries, 2048
    wl = synth.toy(seed=13, batch=2, queries=S, ctx=ctx, topk=K, steps=3)
    gw = GpuWorkload(wl)
    rng = np.random.default_rng(1300 + S)
    base = [None] * wl.batch
    for step in range(3):
        _, _, ctx_lens = gw.inputs(step)
        tk = np.empty((wl.batch, S, K), np.int32)
        for b in range(wl.batch):
            span = int(ctx_lens[b]) - S + 1  # every query sees these tokens
            if base[b] is None:
                base[b] = rng.choice(span, 2600, replace=False)
            else:
                keep = rng.choice(base[b], 2080, replace=False)
                fresh = np.setdiff1d(rng.choice(span, 1200, replace=False), keep)[:520]
                base[b] = np.concatenate([keep, fresh])
            for j in range(S):
                tk[b, j] = np.sort(rng.choice(base[b], K, replace=False))
        print(f"[resolver paths S={S}] step {step} contexts {ctx_lens.tolist()}", flush=True)
        rows_dev, stats_dev = gw.gpu_resolve(torch.from_numpy(tk).to(gw.dev), ctx_lens)
        rows, stats = rows_dev.cpu().numpy(), stats_dev.cpu().numpy()
        for b in range(wl.batch):
            rows_ref, _, st_ref = gw.oracle_resolve(b, tk[b])
            assert np.array_equal(rows[b], rows_ref), f"row ids differ, request {b} step {step}"
            assert tuple(int(x) for x in stats[b]) == st_ref, f"stats {stats[b]} vs {st_ref}"
            check_content(gw, b, rows[b].ravel(), tk[b].ravel())
        st_tok, st_stamp, t2s, _ = gw.ctx.hot_state()
        for b in range(wl.batch):
            o = gw.states[b]
            assert np.array_equal(st_tok[b], o.slot_token), f"slot_token request {b}"
            assert np.array_equal(st_stamp[b], o.slot_stamp), f"slot_stamp request {b}"
            assert np.array_equal(t2s[b], o.tok2slot), f"tok2slot request {b}"
        assert gw.ctx.device_error() == 0
    gw.close()


def test_config1_bf16_8k():
    wl = synth.config(1)
    gw = GpuWorkload(wl)
    run_isolated(gw, 1, label="ctx8k_b1_bf16")
    gw.close()
