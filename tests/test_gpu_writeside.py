"""GPU parity of the host-pool write side: materialised pages hold their rows bit for bit,
releases follow the oracle's rules, and decode steps after the release (with the freed GPU
blocks overwritten) still match the oracle, the released pages' tokens now arriving through
the hot buffer from their host copies."""
import numpy as np
import pytest
import torch

import oracle
import synth
from hs_harness import GpuWorkload
from test_gpu_parity import run_isolated

pytestmark = pytest.mark.gpu

BLOCK = 64


@pytest.mark.parametrize("kv_dtype", [1, 0], ids=["fp8_rows", "bf16_rows"])
def test_materialize_release_then_decode(kv_dtype):
    wl = synth.toy(seed=41, batch=2, queries=2, ctx=(3000, 4100), topk=64, n_layers=2, steps=3,
                   residency=[(synth.RES_HYBRID, 0.6)] * 2, kv_dtype=kv_dtype)
    lay0 = synth.make_layout(wl)
    # complete resident pages (not the tail) to materialise: three per request
    pages = []
    for b in range(wl.batch):
        tail = (int(wl.ctx[b]) - 1) // BLOCK
        res = [int(p) for p in np.nonzero(lay0.block_table[b] >= 0)[0] if p < tail]
        pages += [(b, res[0]), (b, res[len(res) // 2]), (b, res[-1])]
    spare0 = lay0.num_host_blocks
    lay = synth.Layout(lay0.block_table.copy(), lay0.host_block_table.copy(), lay0.idx_block_table,
                       lay0.hot_blocks, lay0.num_gpu_blocks, spare0 + len(pages), lay0.num_idx_blocks)
    gw = GpuWorkload(wl, layout=lay)
    rb = wl.row_bytes
    host = gw.ctx.host_pool.reshape(wl.n_layers, lay.num_host_blocks * BLOCK, rb)
    host[:, spare0 * BLOCK:] = 0  # the new host blocks start empty
    for k, (b, p) in enumerate(pages):
        lay.host_block_table[b, p] = spare0 + k
    gw.ctx.host_block_table.copy_(torch.from_numpy(lay.host_block_table))

    pages_dev = torch.tensor(pages, dtype=torch.int32, device=gw.dev)
    print("[write side] materialise", len(pages), "pages", flush=True)
    gw.ctx.materialize_pages(pages_dev)
    torch.cuda.synchronize()
    assert gw.ctx.device_error() == 0
    gpu_rows = gw.ctx.kv_pool.view(wl.n_layers, lay.num_gpu_blocks * BLOCK, rb).cpu().numpy()
    want = np.zeros_like(host)
    want[:, :spare0 * BLOCK] = host[:, :spare0 * BLOCK]
    oracle.materialize_pages(gpu_rows, want, lay.block_table, lay.host_block_table, pages, wl.n_layers)
    assert np.array_equal(host, want), "host pool differs from the oracle's materialisation"
    for b, p in pages:
        h = lay.host_block_table[b, p]
        for layer in range(wl.n_layers):
            ref = synth.latent_tokens(wl, b, layer, np.arange(p * BLOCK, (p + 1) * BLOCK))
            assert np.array_equal(host[layer, h * BLOCK:(h + 1) * BLOCK], ref)

    # release: the materialised pages, one of them twice, plus the tail page of request 0 and
    # a resident page with no host copy (both refused)
    tail0 = (int(wl.ctx[0]) - 1) // BLOCK
    nohost = [int(p) for p in np.nonzero((lay.block_table[1] >= 0) & (lay.host_block_table[1] < 0))[0]
              if p < (int(wl.ctx[1]) - 1) // BLOCK][0]
    rel = pages + [pages[0], (0, tail0), (1, nohost)]
    rel_dev = torch.tensor(rel, dtype=torch.int32, device=gw.dev)
    lens_dev = torch.from_numpy(np.asarray(wl.ctx, np.int32)).to(gw.dev)
    freed_dev = torch.full((len(rel),), -7, dtype=torch.int32, device=gw.dev)
    print("[write side] release", len(rel), "entries", flush=True)
    gw.ctx.release_pages(rel_dev, lens_dev, freed_dev)
    torch.cuda.synchronize()
    err = gw.ctx.device_error()
    assert err == synth_err(), f"device error {err:#x}"
    freed_ref = oracle.release_pages(lay.block_table, lay.host_block_table, rel, wl.ctx)
    freed = freed_dev.cpu().numpy().tolist()
    # the duplicate entry: either of the two copies gives the block up, the other reports -1
    assert sorted(freed) == sorted(freed_ref), (freed, freed_ref)
    assert freed[len(pages) + 1:] == [-1, -1]
    assert np.array_equal(gw.ctx.block_table.cpu().numpy(), lay.block_table)

    # the freed GPU blocks are reused by someone else: overwrite them
    kv = gw.ctx.kv_pool.view(wl.n_layers, lay.num_gpu_blocks, BLOCK * rb)
    for g in freed_ref:
        if g >= 0:
            kv[:, g] = 0x5A
    torch.cuda.synchronize()
    run_isolated(gw, 3, label="after release")
    gw.close()


def synth_err() -> int:
    from sparse_mla_attention_score_amd import hisparse as hsb
    return hsb.HS_DEVERR_TAIL_PAGE | hsb.HS_DEVERR_NO_HOST_COPY
