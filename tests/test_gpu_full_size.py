"""Parity at the full sizes of the synthetic workloads, in the launch configuration the
benchmark times (the same context configuration and batch), checked against the oracle on
sampled requests.

Per step: the GPU top-K of each sampled request is checked against the oracle's scores; the
GPU resolver runs on the GPU top-K of the whole batch, and for each sampled request the
oracle's LRU state machine, fed the same top-K, must give the same row ids, stats and hot
state bit for bit; every resolved row of a sampled request must hold its token's bytes; the
decode of every layer is checked against dense softmax attention over the same selection.
"""
import numpy as np
import pytest
import torch

import synth
from hs_harness import GpuWorkload, check_attention, check_content, check_topk

pytestmark = pytest.mark.gpu


def run_sampled(wl: synth.Workload, steps: int, sample: list):
    gw = GpuWorkload(wl, verbose=True)
    B, S, K = wl.batch, wl.queries, wl.topk
    worst = 0.0
    for step in range(steps):
        print(f"[{wl.name}] step {step}: GPU calls", flush=True)
        qidx, q, lens = gw.inputs(step)
        tk_dev = gw.gpu_topk(qidx, lens)
        rows_dev, stats_dev = gw.gpu_resolve(tk_dev, lens)
        outs = [gw.gpu_decode(layer, q, rows_dev, lens) for layer in range(wl.n_layers)]
        torch.cuda.synchronize()
        assert gw.ctx.device_error() == 0
        tk = tk_dev.cpu().numpy()
        rows, stats = rows_dev.cpu().numpy(), stats_dev.cpu().numpy()
        st_tok, st_stamp, t2s, req_step = gw.ctx.hot_state(sample)
        for i, b in enumerate(sample):
            print(f"[{wl.name}] step {step}: request {b} (context {int(lens[b])})", flush=True)
            _, sc = gw.oracle_topk(b, qidx, int(lens[b]))
            for j in range(S):
                check_topk(tk[b, j], sc[j], K)
            rows_ref, _, st_ref = gw.oracle_resolve(b, tk[b])
            assert np.array_equal(rows[b], rows_ref), f"row ids differ, request {b} step {step}"
            assert tuple(int(x) for x in stats[b]) == st_ref, f"stats {stats[b]} vs {st_ref}"
            o = gw.states[b]
            assert np.array_equal(st_tok[i], o.slot_token), f"slot_token request {b}"
            assert np.array_equal(st_stamp[i], o.slot_stamp), f"slot_stamp request {b}"
            assert np.array_equal(t2s[i], o.tok2slot), f"tok2slot request {b}"
            assert req_step[i] == step + 1
            check_content(gw, b, rows[b].ravel(), tk[b].ravel())
            for layer, (out, lse) in enumerate(outs):
                for j in range(S):
                    toks = tk[b, j][tk[b, j] >= 0]
                    o_ref, l_ref = gw.oracle_attention(b, j, layer, toks, q)
                    got = out[b, j].float().cpu().numpy().astype(np.float64)
                    worst = max(worst, check_attention(got, lse[b, j].cpu().numpy().astype(np.float64),
                                                       o_ref, l_ref))
        print(f"[{wl.name}] step {step}: misses {int(stats[:, 2].sum())}, hits {int(stats[:, 1].sum())}",
              flush=True)
    print(f"[{wl.name}] worst relative L2 {worst:.2e}", flush=True)
    gw.close()


def test_full_ctx128k_b64_mtp3():
    # the benchmark's workload and context configuration (3 warm-up, 16 timed and 16
    # instrumented steps)
    wl = synth.config(3, steps=35)
    # five steps: from the second on the selections come from the sweep's candidate list
    run_sampled(wl, 5, [0, 21, 37, 63])


def test_full_ctx64k_b32():
    wl = synth.config(2)
    run_sampled(wl, 3, [0, 31])


def test_full_ctx1m_b1_prefix_only():
    wl = synth.config(4)
    run_sampled(wl, 3, [0])


def test_full_mixed_b128_indexshare4():
    wl = synth.config(5)
    lens = np.asarray(wl.ctx)
    kinds = [r[0] for r in wl.residency]
    sample = {int(np.argmax(lens)), int(np.argmin(lens))}
    for k in (synth.RES_FULL, synth.RES_HYBRID, synth.RES_PREFIX):
        idx = [b for b in range(wl.batch) if kinds[b] == k]
        if idx:
            sample.add(max(idx, key=lambda b: lens[b]))
    run_sampled(wl, 2, sorted(sample))
