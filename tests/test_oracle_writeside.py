"""Pins of the oracle's host-pool write side (materialise completed pages, then release them).

The copied bytes are checked against the seeded generator, which regenerates any token's
stored row on its own (not against the oracle's slicing), and the release rules against hand
cases; an end-to-end case follows a released page's tokens through the oracle's resolver.
"""
import numpy as np
import pytest

import oracle
import synth

BLOCK = 64


def spare_host_blocks(lay: synth.Layout, pages) -> synth.Layout:
    """A copy of `lay` in which the given resident pages also own a new host block each."""
    hbt = lay.host_block_table.copy()
    n = lay.num_host_blocks
    for b, p in pages:
        assert lay.block_table[b, p] >= 0 and hbt[b, p] < 0
        hbt[b, p] = n
        n += 1
    return synth.Layout(lay.block_table.copy(), hbt, lay.idx_block_table, lay.hot_blocks,
                        lay.num_gpu_blocks, n, lay.num_idx_blocks)


def workload(kv_dtype=1, n_layers=2):
    wl = synth.toy(seed=31, batch=2, queries=1, ctx=(1000, 1500), topk=16, steps=1,
                   residency=[(synth.RES_HYBRID, 0.5)] * 2, kv_dtype=kv_dtype, n_layers=n_layers)
    return wl, synth.make_layout(wl)


def pools(wl, lay, empty_host_blocks=()):
    """GPU and host pools filled by the generator.  The host blocks listed in
    `empty_host_blocks` are then zeroed: blocks newly assigned to resident pages hold nothing
    until the pages are materialised (the generator writes every host block of the table)."""
    rb = wl.row_bytes
    gpu = np.zeros(wl.n_layers * lay.num_gpu_blocks * BLOCK * rb, np.uint8)
    host = np.zeros(wl.n_layers * lay.num_host_blocks * BLOCK * rb, np.uint8)
    synth.fill_kv(wl, lay, gpu, host if host.size else None)
    host = host.reshape(wl.n_layers, lay.num_host_blocks * BLOCK, rb)
    for h in empty_host_blocks:
        host[:, h * BLOCK:(h + 1) * BLOCK] = 0
    return gpu.reshape(wl.n_layers, lay.num_gpu_blocks * BLOCK, rb), host


def new_host_blocks(lay, pages):
    return [int(lay.host_block_table[b, p]) for b, p in pages]


@pytest.mark.parametrize("kv_dtype", [0, 1])
def test_materialized_rows_are_the_tokens_rows(kv_dtype):
    wl, lay0 = workload(kv_dtype)
    # resident pages that are complete (not the tail), two per request
    pages = []
    for b in range(wl.batch):
        tail = (int(wl.ctx[b]) - 1) // BLOCK
        res = [p for p in np.nonzero(lay0.block_table[b] >= 0)[0] if p < tail]
        pages += [(b, int(res[0])), (b, int(res[-1]))]
    lay = spare_host_blocks(lay0, pages)
    gpu, host = pools(wl, lay, new_host_blocks(lay, pages))
    before = host.copy()
    for b, p in pages:  # the new host blocks start empty
        h = lay.host_block_table[b, p]
        assert not host[:, h * BLOCK:(h + 1) * BLOCK].any()
    oracle.materialize_pages(gpu, host, lay.block_table, lay.host_block_table, pages, wl.n_layers)
    touched = np.zeros(host.shape[1], bool)
    for b, p in pages:
        h = lay.host_block_table[b, p]
        touched[h * BLOCK:(h + 1) * BLOCK] = True
        toks = np.arange(p * BLOCK, (p + 1) * BLOCK)
        for layer in range(wl.n_layers):
            ref = synth.latent_tokens(wl, b, layer, toks)
            assert np.array_equal(host[layer, h * BLOCK:(h + 1) * BLOCK], ref), (b, p, layer)
    # every other host row is untouched
    assert np.array_equal(host[:, ~touched], before[:, ~touched])


def test_materialize_skips_pages_without_a_host_block():
    wl, lay = workload()
    gpu, host = pools(wl, lay)
    before = host.copy()
    b = 0
    p = int(np.nonzero(lay.block_table[b] >= 0)[0][0])  # resident, no host block
    oracle.materialize_pages(gpu, host, lay.block_table, lay.host_block_table, [(b, p)], wl.n_layers)
    assert np.array_equal(host, before)


def test_release_rules():
    bt = np.array([[5, 6, 7, 8, -1]], np.int32)
    hbt = np.array([[0, -1, 2, 3, 4]], np.int32)
    lens = [4 * BLOCK + 1]  # tokens 0 .. 256: the tail page is page 4
    freed = oracle.release_pages(bt, hbt, [(0, 0), (0, 1), (0, 2), (0, 2), (0, 3), (0, 4)], lens)
    # page 0: given up; page 1: no host copy, kept; page 2 listed twice: given up once;
    # page 3: given up; page 4: the tail page (here also host-only), refused
    assert freed == [5, -1, 7, -1, 8, -1]
    assert bt.tolist() == [[-1, 6, -1, -1, -1]]
    # the tail page keeps its GPU block even with a host copy
    bt2 = np.array([[5, 6]], np.int32)
    hbt2 = np.array([[0, 1]], np.int32)
    assert oracle.release_pages(bt2, hbt2, [(0, 1), (0, 0)], [BLOCK + 10]) == [-1, 5]
    assert bt2.tolist() == [[-1, 6]]
    # a page past the context is refused as well
    assert oracle.release_pages(np.array([[1, 2, 3]], np.int32), np.array([[0, 1, 2]], np.int32),
                                [(0, 2)], [BLOCK + 1]) == [-1]


def test_released_page_resolves_to_its_rows_from_the_host_copy():
    # materialise and release a resident prefix page; the resolver then treats its tokens as
    # misses whose host rows are exactly the rows the page held on the GPU
    wl, lay0 = workload()
    b = 1
    tail = (int(wl.ctx[b]) - 1) // BLOCK
    p = int([q for q in np.nonzero(lay0.block_table[b] >= 0)[0] if q < tail][0])
    lay = spare_host_blocks(lay0, [(b, p)])
    gpu, host = pools(wl, lay, new_host_blocks(lay, [(b, p)]))
    oracle.materialize_pages(gpu, host, lay.block_table, lay.host_block_table, [(b, p)], wl.n_layers)
    g = int(lay.block_table[b, p])
    assert oracle.release_pages(lay.block_table, lay.host_block_table, [(b, p)], wl.ctx) == [g]
    toks = np.arange(p * BLOCK + 3, p * BLOCK + 3 + wl.topk, dtype=np.int32)
    st = oracle.HotState.cold(wl.hot_rows, wl.max_pages * BLOCK)
    rows, copies, stats = oracle.resolve(toks[None, :], lay.block_table[b], lay.host_block_table[b],
                                         lay.hot_blocks[b], st)
    assert stats[0] == 0 and stats[2] == len(toks)  # no resident token, all misses
    for token, slot, host_row, dst_row in copies:
        for layer in range(wl.n_layers):
            ref = synth.latent_tokens(wl, b, layer, [token])[0]
            assert np.array_equal(host[layer, host_row], ref)
            assert np.array_equal(gpu[layer, g * BLOCK + token % BLOCK], ref)
