"""GPU parity of hot-page leasing, per-request release and plan windows against the oracle.

Part 1, "How it works": hot pages are leased from the same pool as resident pages when a request
first needs them and given back when it no longer does; a freed block becomes another request's
hot capacity.  Part 1, "Composing with the rest of vLLM": per-step resolver plans that can be
replayed and share the request's hot state.

Stage-isolated like test_gpu_parity.py: the resolver gets the oracle's top-K; row ids, stats,
hot-buffer state, the hot-page tables and the free-block pool must match the oracle bit for bit;
every resolved row holds its token's bytes; attention matches the oracle's dense softmax.
"""
import numpy as np
import pytest
import torch

import synth
from hs_harness import GpuWorkload, check_attention, check_content, check_topk

pytestmark = pytest.mark.gpu


def _topk_ref(gw: GpuWorkload, step: int):
    wl = gw.wl
    qidx, q, lens = gw.inputs(step)
    tk_gpu = gw.gpu_topk(qidx, lens).cpu().numpy()
    tk_ref = np.empty_like(tk_gpu)
    for b in range(wl.batch):
        ref, sc = gw.oracle_topk(b, qidx, int(lens[b]))
        tk_ref[b] = ref
        for j in range(wl.queries):
            check_topk(tk_gpu[b, j], sc[j], wl.topk)
    return q, lens, tk_ref


def _check_state(gw: GpuWorkload, label: str):
    st_tok, st_stamp, t2s, req_step = gw.ctx.hot_state()
    for b in range(gw.wl.batch):
        o = gw.states[b]
        assert np.array_equal(st_tok[b], o.slot_token), f"{label}: slot_token request {b}"
        assert np.array_equal(st_stamp[b], o.slot_stamp), f"{label}: slot_stamp request {b}"
        assert np.array_equal(t2s[b], o.tok2slot), f"{label}: tok2slot request {b}"
        assert req_step[b] == o.step, f"{label}: step request {b}"
    if gw.leasing:
        assert np.array_equal(gw.ctx.hot_blocks.cpu().numpy(), gw.hot), f"{label}: hot-page tables"
        assert gw.ctx.pool_free() == list(gw.pool.free), f"{label}: free-block pool"


def _resolve_and_check(gw: GpuWorkload, q, lens, tk_ref, label: str, begin=None, window=None):
    """Resolve on both sides (begin: per-request window flags, window: the oracle's window
    starts), compare, decode and check attention.  Returns the GPU row ids (device) and the
    decode output (device)."""
    wl = gw.wl
    bw = None if begin is None else torch.tensor(begin, dtype=torch.int32, device=gw.dev)
    rows_dev = torch.empty((wl.batch, wl.queries, wl.topk), dtype=torch.int32, device=gw.dev)
    stats_dev = torch.empty((wl.batch, 4), dtype=torch.int32, device=gw.dev)
    gw.ctx.resolve(torch.from_numpy(tk_ref).to(gw.dev), gw.to_dev(lens), rows_dev, stats_dev, bw)
    rows, stats = rows_dev.cpu().numpy(), stats_dev.cpu().numpy()
    for b in range(wl.batch):
        ws = None if window is None else window[b]
        rows_ref, _, st_ref = gw.oracle_resolve(b, tk_ref[b], ws)
        assert np.array_equal(rows[b], rows_ref), f"{label}: row ids differ, request {b}"
        assert tuple(int(x) for x in stats[b]) == st_ref, f"{label}: stats {stats[b]} vs {st_ref}"
    _check_state(gw, label)
    for b in range(wl.batch):
        check_content(gw, b, rows[b].ravel(), tk_ref[b].ravel())
    out, lse = gw.gpu_decode(0, q, rows_dev, lens)
    o64 = out.float().cpu().numpy().astype(np.float64)
    l64 = lse.cpu().numpy().astype(np.float64)
    for b in range(wl.batch):
        for j in range(wl.queries):
            toks = tk_ref[b, j][tk_ref[b, j] >= 0]
            o_ref, l_ref = gw.oracle_attention(b, j, 0, toks, q)
            check_attention(o64[b, j], l64[b, j], o_ref, l_ref)
    return rows_dev, out


def _release(gw: GpuWorkload, reqs, label: str):
    gw.ctx.hot_release(torch.tensor(reqs, dtype=torch.int32, device=gw.dev))
    for b in reqs:
        gw.oracle_release(b)
    _check_state(gw, label)


def test_leased_hot_pages_across_requests():
    # three requests share 28 free blocks for up to 3 x 12 hot pages: before a call, requests
    # are released (most pages first) until the pool covers what the call could lease, and
    # their blocks are leased again by the others
    wl = synth.toy(seed=31, batch=3, queries=2, ctx=(3000, 2200, 4100), topk=256, steps=8,
                   residency=[(synth.RES_HYBRID, 0.25), (synth.RES_PREFIX, 0.0),
                              (synth.RES_HYBRID, 0.1)])
    lay = synth.make_layout(wl)
    rng = np.random.default_rng(31)
    initial = [int(x) for x in rng.permutation(lay.hot_blocks.ravel())[:28]]
    gw = GpuWorkload(wl, layout=lay, lease_pool=initial)
    assert (gw.ctx.hot_blocks.cpu().numpy() == -1).all()
    _check_state(gw, "start")
    pages = gw.wl.hot_rows // 64
    per_call = (wl.queries * wl.topk) // 64 + 1        # pages one call can lease per request

    def could_lease(b):
        return min(per_call, pages - int((gw.hot[b] != -1).sum()))

    released = 0
    for step in range(wl.steps):
        print(f"[leasing] step {step}", flush=True)
        q, lens, tk_ref = _topk_ref(gw, step)
        out = []
        while len(gw.pool.free) + sum(int((gw.hot[b] != -1).sum()) for b in out) < \
                sum(per_call if b in out else could_lease(b) for b in range(wl.batch)):
            b = max((x for x in range(wl.batch) if x not in out),
                    key=lambda x: int((gw.hot[x] != -1).sum()))
            out.append(b)
        if out:
            _release(gw, out, f"release {out} before step {step}")
            released += len(out)
        _resolve_and_check(gw, q, lens, tk_ref, f"step {step}")
        held = [int(x) for x in gw.hot.ravel() if x != -1]
        assert sorted(held + list(gw.pool.free)) == sorted(initial)
    assert released > 0
    # two requests released together, one of them listed twice: blocks return once, in order
    _release(gw, [2, 0, 2], "release 2, 0, 2")
    assert gw.ctx.device_error() == 0
    gw.close()


def test_release_is_a_per_request_reset():
    # static hot pages: releasing one request slot makes only that request cold; the others keep
    # their hot state, and the released one refetches its rows as misses (a new request in the
    # slot would find none of the old request's tokens)
    wl = synth.toy(seed=32, batch=3, queries=1, ctx=(2600, 3100, 1900), topk=256, steps=5,
                   residency=[(synth.RES_PREFIX, 0.0)] * 3)
    gw = GpuWorkload(wl)
    for step in range(wl.steps):
        print(f"[release] step {step}", flush=True)
        q, lens, tk_ref = _topk_ref(gw, step)
        if step == 3:
            before = gw.ctx.hot_state()
            _release(gw, [1], "release 1")
            after = gw.ctx.hot_state()
            for b in (0, 2):
                assert np.array_equal(before[0][b], after[0][b]) and np.array_equal(before[2][b], after[2][b])
            assert (after[0][1] == -1).all() and (after[2][1] == -1).all() and after[3][1] == 0
            assert np.array_equal(gw.ctx.hot_blocks.cpu().numpy(), gw.lay.hot_blocks)
        _resolve_and_check(gw, q, lens, tk_ref, f"step {step}")
    assert gw.ctx.device_error() == 0
    gw.close()


def test_plan_windows_replay():
    # per-request windows of 1-2 calls: inside a window no slot an earlier call of the window
    # touched is reused, so the window's first plan can be replayed at its end and gives the same
    # attention bit for bit
    wl = synth.toy(seed=33, batch=2, queries=1, ctx=(5000, 3500), topk=256, steps=9,
                   residency=[(synth.RES_PREFIX, 0.0), (synth.RES_HYBRID, 0.2)])
    gw = GpuWorkload(wl)
    rng = np.random.default_rng(33)
    window = [0, 0]
    first = None      # (q, lens, rows of the window's first call, its output) of request 0's window
    replays = 0
    for step in range(wl.steps):
        q, lens, tk_ref = _topk_ref(gw, step)
        begin = [1 if step == 0 or rng.random() < 0.5 else 0 for _ in range(wl.batch)]
        if step % 2 == 0:
            begin[0] = 1                                        # request 0: windows of two calls
        else:
            begin[0] = 0
        if begin[0] and first is not None:
            q0, l0, r0, o0 = first                              # replay before the window ends
            out, _ = gw.gpu_decode(0, q0, r0, l0)
            assert torch.equal(out.view(torch.int16)[0], o0.view(torch.int16)[0]), f"replay at {step}"
            replays += 1
        for b in range(wl.batch):
            if begin[b]:
                window[b] = gw.states[b].step
        print(f"[windows] step {step} begin {begin}", flush=True)
        rows, out = _resolve_and_check(gw, q, lens, tk_ref, f"step {step}", begin=begin,
                                       window=list(window))
        if begin[0]:
            first = (q, lens, rows.clone(), out.clone())
    assert replays >= 3
    assert gw.ctx.device_error() == 0
    gw.close()


def test_pool_argument_errors():
    import sparse_mla_attention_score_amd.hisparse as hsb
    wl = synth.toy(seed=34, batch=1, queries=1, ctx=(900,), topk=64, steps=1)
    gw = GpuWorkload(wl)
    blocks = torch.tensor([1, 2], dtype=torch.int32, device=gw.dev)
    with pytest.raises(hsb.HiSparseError):                      # no leasing on this context
        gw.ctx.pool_give(blocks)
    with pytest.raises(hsb.HiSparseError):
        hsb.hs_hot_release(gw.ctx.ctx, 0, 2, gw.ctx.stream())
    gw.ctx.hot_release(torch.tensor([5], dtype=torch.int32, device=gw.dev))   # outside max_batch
    assert gw.ctx.device_error() == hsb.HS_DEVERR_BAD_REQUEST
    gw.close()
