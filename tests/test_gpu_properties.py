"""GPU properties that hold at any size: repeat runs are bitwise identical, where a row lives
(resident, hot, copied in on a miss) does not change any result, a HIP-graph replay of the
step equals eager execution, device-side faults forced from the host are flagged without
touching memory outside the buffers, and per-kernel timing counts each launch."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_score_amd.hisparse as hsb
import synth
from hs_harness import GpuWorkload, check_attention, check_topk

pytestmark = pytest.mark.gpu


def _step(gw: GpuWorkload, step: int, layers=None):
    """One eager step through the three calls; (top-K, row ids, stats, [(out, lse) per layer])."""
    qidx, q, lens = gw.inputs(step)
    tk = gw.gpu_topk(qidx, lens)
    rows, stats = gw.gpu_resolve(tk, lens)
    outs = []
    for layer in (range(gw.wl.n_layers) if layers is None else layers):
        o, l = gw.gpu_decode(layer, q, rows, lens)
        outs.append((o.view(torch.int16).cpu().numpy(), l.cpu().numpy()))
    torch.cuda.synchronize()
    return tk.cpu().numpy(), rows.cpu().numpy(), stats.cpu().numpy(), outs


def test_repeat_runs_are_bitwise_identical():
    wl = synth.toy(seed=21, batch=3, queries=4, ctx=(5000, 2600, 3100), topk=256, steps=3)
    print(f"[determinism] {wl.name}", flush=True)
    a, b = GpuWorkload(wl), GpuWorkload(wl)
    for step in range(3):
        ra, rb = _step(a, step), _step(b, step)
        assert np.array_equal(ra[0], rb[0]) and np.array_equal(ra[1], rb[1])
        assert np.array_equal(ra[2], rb[2])
        for (oa, la), (ob, lb) in zip(ra[3], rb[3]):
            assert np.array_equal(oa, ob) and np.array_equal(la.view(np.int32), lb.view(np.int32))
    assert a.ctx.device_error() == 0 and b.ctx.device_error() == 0
    a.close()
    b.close()


def test_results_do_not_depend_on_residency():
    # the same requests with every page resident, with 25 % resident (hot hits and misses),
    # and with only the tail page resident: identical top-K and attention, bit for bit
    kinds = {"full": (synth.RES_FULL, 1.0), "hybrid": (synth.RES_HYBRID, 0.25),
             "prefix": (synth.RES_PREFIX, 0.0)}
    runs = {}
    for name, res in kinds.items():
        wl = synth.toy(seed=22, batch=2, queries=2, ctx=(6000, 3300), topk=512, n_layers=2,
                       residency=[res, res], steps=3)
        print(f"[residency] {name}", flush=True)
        gw = GpuWorkload(wl)
        runs[name] = [_step(gw, s) for s in range(3)]
        assert gw.ctx.device_error() == 0
        gw.close()
    for name in ("hybrid", "prefix"):
        for s in range(3):
            ref, got = runs["full"][s], runs[name][s]
            assert np.array_equal(ref[0], got[0]), f"top-K differs ({name}, step {s})"
            for (o0, l0), (o1, l1) in zip(ref[3], got[3]):
                assert np.array_equal(o0, o1), f"attention differs ({name}, step {s})"
                assert np.array_equal(l0.view(np.int32), l1.view(np.int32))
    # the residency really differed: the prefix run copied rows in, the full run did not
    assert runs["full"][0][2][:, 2].sum() == 0
    assert runs["prefix"][0][2][:, 2].sum() > 0


def test_graph_replay_matches_eager():
    wl = synth.toy(seed=23, batch=2, queries=4, ctx=(4200, 3000), topk=256, n_layers=2, steps=4)
    print(f"[graph] {wl.name}", flush=True)
    eager, graphed = GpuWorkload(wl), GpuWorkload(wl)
    B, S, K, dev = wl.batch, wl.queries, wl.topk, graphed.dev
    qidx0, q0, lens0 = graphed.inputs(0)
    s_qidx = graphed.to_dev(qidx0).clone()
    s_q = graphed.to_dev(q0).clone()
    s_lens = graphed.to_dev(lens0).clone()
    s_tk = torch.empty((B, S, K), dtype=torch.int32, device=dev)
    s_rows = torch.empty_like(s_tk)
    s_stats = torch.empty((B, 4), dtype=torch.int32, device=dev)
    s_out = [torch.empty((B, S, 64, 512), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    s_lse = [torch.empty((B, S, 64), dtype=torch.float32, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.ctx.index_topk(s_qidx, graphed.w, s_lens, s_tk)
        graphed.ctx.resolve(s_tk, s_lens, s_rows, s_stats)
        for layer in range(2):
            graphed.ctx.decode(layer, s_q, s_rows, s_lens, graphed.sm_scale, s_out[layer], s_lse[layer])
    torch.cuda.synchronize()
    for step in range(4):
        qidx, q, lens = graphed.inputs(step)
        s_qidx.copy_(graphed.to_dev(qidx))
        s_q.copy_(graphed.to_dev(q))
        s_lens.copy_(graphed.to_dev(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _step(eager, step)
        assert np.array_equal(s_tk.cpu().numpy(), ref[0]), f"top-K, replay {step}"
        assert np.array_equal(s_rows.cpu().numpy(), ref[1]), f"row ids, replay {step}"
        assert np.array_equal(s_stats.cpu().numpy(), ref[2]), f"stats, replay {step}"
        for layer in range(2):
            assert np.array_equal(s_out[layer].view(torch.int16).cpu().numpy(), ref[3][layer][0])
            assert np.array_equal(s_lse[layer].cpu().numpy().view(np.int32), ref[3][layer][1].view(np.int32))
    assert graphed.ctx.device_error() == 0 and eager.ctx.device_error() == 0
    del g
    eager.close()
    graphed.close()


def test_forced_faults_are_flagged():
    import sparse_mla_attention_score_amd.hisparse as hsb
    wl = synth.toy(seed=24, batch=3, queries=2, ctx=(3000, 900, 2000), topk=1024,
                   residency=[(synth.RES_HYBRID, 0.25)] * 3, steps=1)
    gw = GpuWorkload(wl)
    lay, ctx = gw.lay, gw.ctx
    qidx, q, lens = gw.inputs(0)

    print("[faults] empty batch", flush=True)
    empty = torch.empty((0, wl.queries, wl.topk), dtype=torch.int32, device=gw.dev)
    hsb.hisparse_index_topk(ctx.ctx, gw.to_dev(qidx).data_ptr(), gw.w.data_ptr(),
                            gw.to_dev(lens).data_ptr(), 0, wl.queries, empty.data_ptr(), ctx.stream())
    assert ctx.device_error() == 0
    with pytest.raises(hsb.HiSparseError):
        hsb.hisparse_index_topk(ctx.ctx, 0, 0, 0, wl.batch, 5, 0, ctx.stream())

    print("[faults] context shorter than the query count", flush=True)
    bad_lens = lens.copy()
    bad_lens[1] = wl.queries - 1
    tk = gw.gpu_topk(qidx, bad_lens).cpu().numpy()
    assert ctx.device_error() & hsb.HS_DEVERR_SHORT_CONTEXT
    assert (tk[1] == -1).all()
    for b in (0, 2):  # the other requests are unaffected
        _, sc = gw.oracle_topk(b, qidx, int(lens[b]))
        for j in range(wl.queries):
            check_topk(tk[b, j], sc[j], wl.topk)

    print("[faults] indexer block id out of range", flush=True)
    saved = ctx.idx_block_table.clone()
    ctx.idx_block_table[0, 3] = lay.num_idx_blocks
    gw.gpu_topk(qidx, lens)
    assert ctx.device_error() & hsb.HS_DEVERR_BAD_BLOCK
    ctx.idx_block_table.copy_(saved)

    print("[faults] placeholder page without a host copy", flush=True)
    # request 1 is shorter than K: every token is selected, so its first non-resident page
    # is requested; remove that page's host block
    b = 1
    page = int(np.nonzero(lay.block_table[b][: (int(lens[b]) + 63) // 64] < 0)[0][0])
    saved_h = ctx.host_block_table.clone()
    ctx.host_block_table[b, page] = -1
    tk = gw.gpu_topk(qidx, lens)
    rows, _ = gw.gpu_resolve(tk, lens)
    out, _ = gw.gpu_decode(0, q, rows, lens)
    torch.cuda.synchronize()
    err = ctx.device_error()
    assert err & hsb.HS_DEVERR_NO_HOST_COPY
    r = rows.cpu().numpy()[b]
    t = tk.cpu().numpy()[b]
    on_page = (t >= page * 64) & (t < page * 64 + 64)
    assert on_page.any() and (r[on_page] == -1).all()
    ctx.host_block_table.copy_(saved_h)
    gw.close()


def test_kernel_timing_counts_each_launch():
    wl = synth.toy(seed=25, batch=2, queries=2, ctx=(2000, 1500), topk=64, n_layers=2, steps=1)
    gw = GpuWorkload(wl)
    gw.ctx.kernel_timing(True)
    _step(gw, 0)
    t = gw.ctx.kernel_times()
    gw.ctx.kernel_timing(False)
    for name in ("index_score", "topk_select", "resolve", "miss_copy"):
        assert t[name][1] == 1, (name, t[name])
    assert t["decode"][1] == 2
    assert all(ms > 0 for ms, n in t.values() if n)
    gw.close()


def test_fp8_decode_ignores_nan_bytes_outside_its_rows():
    # Block 0 of the pool is never used and holds NaN codes (0xFF) and a NaN scale in every
    # row.  A short context (97 rows: a partial 64-row tile) and row ids replaced by -1 in the
    # middle of a list must still give the oracle's output over the remaining rows.
    wl = synth.toy(seed=26, batch=2, queries=1, ctx=(97, 300), topk=128, steps=1,
                   residency=[(synth.RES_FULL, 1.0)] * 2)
    lay = synth.make_layout(wl)
    lay.block_table[lay.block_table >= 0] += 1
    lay.hot_blocks = lay.hot_blocks + 1
    lay.num_gpu_blocks += 1
    print("[nan pool] build", flush=True)
    gw = GpuWorkload(wl, layout=lay)
    kv = gw.ctx.kv_pool.view(wl.n_layers, lay.num_gpu_blocks, 64 * wl.row_bytes)
    kv[:, 0] = 0xFF
    torch.cuda.synchronize()
    qidx, q, lens = gw.inputs(0)
    tk = gw.gpu_topk(qidx, lens)
    rows, _ = gw.gpu_resolve(tk, lens)
    rows_np = rows.cpu().numpy()
    tk_np = tk.cpu().numpy()
    drop = {1: [5, 17, 100]}  # request 1: three entries skipped
    for b, idx in drop.items():
        rows_np[b, 0, idx] = -1
    rows_cut = torch.from_numpy(rows_np).to(gw.dev)
    out, lse = gw.gpu_decode(0, q, rows_cut, lens)
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    # a -1 inside a query's range is an invalid row id: flagged, and left out of the softmax
    assert gw.ctx.device_error() == hsb.HS_DEVERR_BAD_ROW
    for b in range(wl.batch):
        keep = tk_np[b, 0] >= 0
        for i in drop.get(b, []):
            keep[i] = False
        o_ref, l_ref = gw.oracle_attention(b, 0, 0, tk_np[b, 0][keep], q)
        assert np.all(np.isfinite(out[b, 0])), f"NaN in request {b}"
        check_attention(out[b, 0], lse[b, 0], o_ref, l_ref)
    gw.close()


def test_two_live_contexts_of_different_shapes():
    # Kernel LDS limits are process-wide: a second, smaller context created while a larger
    # one is alive must not break it.  The wide context also resolves one query at a time
    # although it is configured for two, on a page table large enough that the one-query
    # layout keeps the page tables in LDS.
    from test_gpu_parity import run_isolated
    big = synth.toy(seed=27, batch=2, queries=4, ctx=(6000, 2600), topk=512, steps=4)
    print("[two contexts] build", flush=True)
    a = GpuWorkload(big)
    small = synth.toy(seed=28, batch=3, queries=1, ctx=(3000, 900, 1400), topk=64, steps=4)
    b = GpuWorkload(small, topk_lds_candidates=1)
    wide = synth.toy(seed=29, batch=1, queries=1, ctx=(5000,), topk=2048, hot_rows=4096, steps=2)
    c = GpuWorkload(wide, max_pages=12000, max_queries=2)
    for gw in (a, b, c):
        gw.steps_done = 0
    for rnd in range(2):
        for name, gw in (("big", a), ("small", b), ("wide", c)):
            print(f"[two contexts] round {rnd} {name}", flush=True)
            run_one_step(gw)
    for gw in (a, b, c):
        assert gw.ctx.device_error() == 0
        gw.close()


def run_one_step(gw: GpuWorkload):
    """Step `gw.steps_done` of a workload in stage-isolated parity with the oracle."""
    from hs_harness import check_attention as _chk
    wl = gw.wl
    step = gw.steps_done
    qidx, q, lens = gw.inputs(step)
    tk_gpu = gw.gpu_topk(qidx, lens).cpu().numpy()
    tk_ref = np.empty_like(tk_gpu)
    for b in range(wl.batch):
        ref, sc = gw.oracle_topk(b, qidx, int(lens[b]))
        tk_ref[b] = ref
        for j in range(wl.queries):
            check_topk(tk_gpu[b, j], sc[j], wl.topk)
    rows_dev, stats_dev = gw.gpu_resolve(torch.from_numpy(tk_ref).to(gw.dev), lens)
    rows, stats = rows_dev.cpu().numpy(), stats_dev.cpu().numpy()
    for b in range(wl.batch):
        rows_ref, _, st_ref = gw.oracle_resolve(b, tk_ref[b])
        assert np.array_equal(rows[b], rows_ref), f"row ids differ, request {b}"
        assert tuple(int(x) for x in stats[b]) == st_ref
    out, lse = gw.gpu_decode(0, q, rows_dev, lens)
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    for b in range(wl.batch):
        for j in range(wl.queries):
            toks = tk_ref[b, j][tk_ref[b, j] >= 0]
            o_ref, l_ref = gw.oracle_attention(b, j, 0, toks, q)
            _chk(out[b, j], lse[b, j], o_ref, l_ref)
    gw.steps_done = step + 1
