"""The seeded input generator: published Philox vectors, encoders, addressability, layouts."""
import numpy as np
import torch

import synth


def test_philox4x32_10_known_answers():
    # Random123 known-answer vectors for philox4x32-10 (counter, key) -> output
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    out = np.zeros(4, np.uint32)
    for ctr, key, expect in kat:
        synth.lib().synth_philox(key[0], key[1], *ctr, out.ctypes.data)
        assert tuple(int(x) for x in out) == expect


def test_encoders_match_torch_casts():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 7, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 448.0, 460.0, 2 ** -10, 2 ** -9 * 1.5])])
    ref8 = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.encode_e4m3(x), ref8)
    refb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.encode_bf16(x), refb)


def test_normals_look_standard():
    z = synth.normals(1, 3, 0, 0, 0, 1 << 18)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


def test_paged_fill_equals_token_order_and_layout_invariants():
    wl = synth.toy(seed=5, batch=3, queries=2, ctx=(200, 333, 64), topk=16, kv_dtype=1,
                   residency=[(synth.RES_HYBRID, 0.25), (synth.RES_FULL, 1.0), (synth.RES_PREFIX, 0.0)])
    lay = synth.make_layout(wl)
    # every page present, the tail page and all future pages GPU-resident,
    # every placeholder page has a host copy, block ids unique
    for b in range(wl.batch):
        n_now = -(-wl.ctx[b] // 64)
        n_all = -(-(wl.ctx[b] + wl.steps * wl.queries) // 64)
        assert np.all(lay.idx_block_table[b, :n_all] >= 0)
        assert np.all(lay.block_table[b, n_now - 1:n_all] >= 0)
        ph = lay.block_table[b, :n_all] < 0
        assert np.all(lay.host_block_table[b, :n_all][ph] >= 0)
        assert np.all(lay.host_block_table[b, :n_all][~ph] == -1)
    used = np.concatenate([lay.block_table[lay.block_table >= 0], lay.hot_blocks.ravel()])
    assert len(np.unique(used)) == len(used) == lay.num_gpu_blocks
    assert np.all(lay.block_table[1, :-(-wl.ctx[1] // 64)] >= 0)               # full residency
    pool = np.zeros(lay.num_idx_blocks * wl.idx_block_bytes, np.uint8)
    synth.fill_idx_pool(wl, lay, pool)
    gpu = np.zeros(lay.num_gpu_blocks * 64 * wl.row_bytes, np.uint8)
    host = np.zeros(lay.num_host_blocks * 64 * wl.row_bytes, np.uint8)
    synth.fill_kv(wl, lay, gpu, host)
    b = 0
    L = wl.ctx[b]
    codes, scale = synth.idx_tokens(wl, b, 0, L)
    rows = synth.latent_tokens(wl, b, 0, np.arange(L))
    for t in range(0, L, 7):
        blk = lay.idx_block_table[b, t // 64]
        base = blk * 8448
        assert np.array_equal(pool[base + (t % 64) * 128: base + (t % 64) * 128 + 128], codes[t])
        assert pool[base + 8192 + (t % 64) * 4: base + 8192 + (t % 64) * 4 + 4].view(np.float32)[0] == scale[t]
        g = lay.block_table[b, t // 64]
        src = gpu if g >= 0 else host
        r = (g if g >= 0 else lay.host_block_table[b, t // 64]) * 64 + t % 64
        assert np.array_equal(src[r * 656:(r + 1) * 656], rows[t])
    assert np.all(rows[:, 644:] == 0)


def test_query_chain_drifts_and_is_reproducible():
    wl = synth.config(2, scale=64, batch=2)
    ch = synth.qidx(wl, 0, 6).astype(np.uint32) << 16
    q = ch.view(np.float32).reshape(6, -1).astype(np.float64)
    c = [np.corrcoef(q[n], q[n + 1])[0, 1] for n in range(5)]
    assert all(0.93 < x < 0.97 for x in c)
    assert np.array_equal(synth.qidx(wl, 0, 6), synth.qidx(wl, 0, 6))
    assert not np.array_equal(synth.qidx(wl, 1, 6), synth.qidx(wl, 0, 6))


def test_config_table():
    c3 = synth.config(3)
    assert (c3.batch, c3.queries, c3.ctx[0], c3.hot_rows, c3.row_bytes, c3.idx_token_bytes) == \
        (64, 4, 131072, 10240, 656, 132)
    c5 = synth.config(5)
    assert c5.n_layers == 4 and c5.batch == 128
    assert 4096 <= min(c5.ctx) and max(c5.ctx) <= 1048576
    assert 15e6 < sum(c5.ctx) < 40e6
    kinds = {r[0] for r in c5.residency}
    assert kinds == {synth.RES_FULL, synth.RES_HYBRID, synth.RES_PREFIX}
