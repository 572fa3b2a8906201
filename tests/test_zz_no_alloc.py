"""sparse_mla_decode_noalloc (the decode for callers that cannot allocate) against
sparse_mla_decode, through the C ABI: two calls in a row, the second smaller, each with split-K
partials in the fixed scratch; outputs bit for bit equal to the workspace entry point's, and
within the attention tolerance of the oracle."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_score_amd.hisparse as hsb
import synth
from hs_harness import GpuWorkload, check_attention

pytestmark = pytest.mark.gpu


def _call_both(gw: GpuWorkload, B: int, S: int, step: int):
    wl = gw.wl
    qidx, q, lens = gw.inputs(step)
    tk = gw.gpu_topk(qidx, lens)
    rows, _ = gw.gpu_resolve(tk, lens)
    qd = gw.to_dev(q)[:B, :S].contiguous()
    rd = rows[:B, :S].contiguous()
    ld = gw.to_dev(lens)[:B].contiguous()
    if S < wl.queries:
        # a call with fewer queries than the step's: query j of the call is query
        # (wl.queries - S + j) of the step, whose rows the shortened context keeps visible
        qd = gw.to_dev(q)[:B, wl.queries - S:].contiguous()
        rd = rows[:B, wl.queries - S:].contiguous()
    splits = hsb.hs_decode_splits(gw.ctx.ctx, B, S)
    assert splits > 1, "the comparison must exercise the split-K scratch"
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, S, 64, 512), float("nan"), dtype=torch.bfloat16, device=gw.dev)
        lse = torch.full((B, S, 64), float("nan"), dtype=torch.float32, device=gw.dev)
        if noalloc:
            gw.ctx.decode_noalloc(0, qd, rd, ld, gw.sm_scale, out, lse)
        else:
            gw.ctx.decode(0, qd, rd, ld, gw.sm_scale, out, lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    (o1, l1), (o2, l2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    tk_np = tk.cpu().numpy()
    o = o2.float().cpu().numpy().astype(np.float64)
    l = l2.cpu().numpy().astype(np.float64)
    j0 = wl.queries - S
    for b in range(B):
        for j in range(S):
            toks = tk_np[b, j0 + j][tk_np[b, j0 + j] >= 0]
            o_ref, l_ref = gw.oracle_attention(b, j0 + j, 0, toks, q)
            check_attention(o[b, j], l[b, j], o_ref, l_ref)
    return splits


def test_noalloc_decode_matches_workspace_decode():
    wl = synth.toy(seed=51, batch=3, queries=2, ctx=(2600, 1900, 3100), topk=512, steps=2)
    gw = GpuWorkload(wl)
    print("[noalloc] 3 x 2 queries", flush=True)
    s1 = _call_both(gw, 3, 2, 0)
    print("[noalloc] 1 x 1 query", flush=True)
    s2 = _call_both(gw, 1, 1, 1)
    assert s1 * 6 <= 512 and s2 <= 512 and s2 >= s1
    assert gw.ctx.device_error() == 0
    gw.close()
