"""Shared helpers for the GPU parity tests: a workload built on the device through the C ABI
binding, the oracle run on the same generated inputs, and the comparison rules.

Comparison rules (readings stated in the design doc):
* top-K: the GPU set must equal the oracle set, except tokens whose float64 oracle score lies
  within 1e-5 relative of the K-th oracle score, which may be swapped; order ascending,
  padding -1;
* resolver: row ids, stats and hot-buffer state bit-exact (the GPU resolver is fed the
  oracle's top-K so both sides decide on the same input);
* attention: |gpu - oracle| <= 1e-2 + 2e-2 |oracle| elementwise, plus a relative-L2
  diagnostic bound.
"""
from __future__ import annotations

import math
import time

import numpy as np
import torch

import oracle
import synth
from sparse_mla_attention_score_amd import hisparse as hsb

TIE_REL = 1e-5
ATOL, RTOL = 1e-2, 2e-2
REL_L2_MAX = 5e-3


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class GpuWorkload:
    def __init__(self, wl: synth.Workload, device: str = "cuda:0", topk_lds_candidates: int = 0,
                 layout: synth.Layout | None = None, verbose: bool = False,
                 max_pages: int | None = None, max_queries: int | None = None,
                 lease_pool: list | None = None, max_batch: int | None = None):
        """`max_pages` / `max_queries` / `max_batch` configure the context wider than the workload
        needs (the block tables are padded with placeholders).  With `lease_pool` (a list of GPU blocks, in
        pool order) hot pages are leased from that free-block pool on first need, on the GPU and
        in the oracle alike, instead of taking the layout's hot blocks."""
        self.wl = wl
        self.lay = layout or synth.make_layout(wl)
        lay = self.lay
        if max_pages is not None and max_pages > lay.block_table.shape[1]:
            pad = ((0, 0), (0, max_pages - lay.block_table.shape[1]))
            lay.block_table = np.pad(lay.block_table, pad, constant_values=-1)
            lay.host_block_table = np.pad(lay.host_block_table, pad, constant_values=-1)
            lay.idx_block_table = np.pad(lay.idx_block_table, pad, constant_values=-1)
        if max_batch is not None and max_batch > lay.block_table.shape[0]:
            pad = ((0, max_batch - lay.block_table.shape[0]), (0, 0))
            lay.block_table = np.pad(lay.block_table, pad, constant_values=-1)
            lay.host_block_table = np.pad(lay.host_block_table, pad, constant_values=-1)
            lay.idx_block_table = np.pad(lay.idx_block_table, pad, constant_values=-1)
            lay.hot_blocks = np.pad(lay.hot_blocks, pad, constant_values=0)
        self.dev = torch.device(device)
        cfg = hsb.make_config(topk=wl.topk, kv_dtype=wl.kv_dtype, idx_dtype=wl.idx_dtype,
                              n_layers=wl.n_layers, max_batch=lay.block_table.shape[0],
                              max_queries=max_queries or wl.queries,
                              max_pages_per_req=lay.block_table.shape[1], hot_rows_per_req=wl.hot_rows,
                              num_gpu_blocks=lay.num_gpu_blocks, num_idx_blocks=lay.num_idx_blocks,
                              num_host_blocks=lay.num_host_blocks,
                              topk_lds_candidates=topk_lds_candidates,
                              hot_leasing=1 if lease_pool is not None else 0)
        self.ctx = hsb.Context(cfg, device)
        t0 = time.time()
        idx_stage = np.zeros(lay.num_idx_blocks * wl.idx_block_bytes, np.uint8)
        synth.fill_idx_pool(wl, lay, idx_stage)
        self.ctx.idx_pool.copy_(torch.from_numpy(idx_stage))
        del idx_stage
        if verbose:
            print(f"[{wl.name}] indexer pool filled ({time.time() - t0:.1f} s)", flush=True)
        # one layer at a time: the staging buffer holds one layer's resident rows
        nb = lay.num_gpu_blocks * 64 * wl.row_bytes
        hb = lay.num_host_blocks * 64 * wl.row_bytes
        kv_stage = np.zeros(nb, np.uint8)
        for layer in range(wl.n_layers):
            if layer:
                kv_stage.fill(0)
            host = self.ctx.host_pool[layer * hb:(layer + 1) * hb] if hb else None
            synth.fill_kv(wl, lay, kv_stage, host, layers=[layer])
            self.ctx.kv_pool[layer * nb:(layer + 1) * nb].copy_(torch.from_numpy(kv_stage))
            if verbose:
                print(f"[{wl.name}] layer {layer} rows filled ({time.time() - t0:.1f} s)", flush=True)
        del kv_stage
        self.ctx.idx_block_table.copy_(torch.from_numpy(lay.idx_block_table))
        self.ctx.block_table.copy_(torch.from_numpy(lay.block_table))
        self.ctx.host_block_table.copy_(torch.from_numpy(lay.host_block_table))
        self.leasing = lease_pool is not None
        self.pool = None
        self.hot = lay.hot_blocks                       # the oracle's hot-page tables
        if self.leasing:
            self.hot = np.full_like(lay.hot_blocks, -1)
            self.pool = oracle.HotPool(lease_pool)
            self.ctx.pool_give(torch.tensor(list(lease_pool), dtype=torch.int32, device=self.dev))
        elif lay.hot_blocks.size:
            self.ctx.hot_blocks.copy_(torch.from_numpy(lay.hot_blocks))
        torch.cuda.synchronize()
        self.chains = [synth.qidx(wl, b, (wl.steps + 1) * wl.queries) for b in range(wl.batch)]
        self.w_np = synth.head_weights(wl)
        self.w = torch.from_numpy(self.w_np).to(self.dev)
        self.sm_scale = 1.0 / math.sqrt(576.0)
        self._keys = {}
        self.states = [oracle.HotState.cold(wl.hot_rows, lay.block_table.shape[1] * 64)
                       for _ in range(wl.batch)]

    # ------------------------------------------------------------ inputs
    def inputs(self, step: int):
        wl = self.wl
        qidx = synth.qidx_step(wl, step, self.chains)
        q = synth.mla_q(wl, step)
        ctx_lens = wl.ctx_at(step).astype(np.int32)
        return qidx, q, ctx_lens

    def to_dev(self, a: np.ndarray) -> torch.Tensor:
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(self.dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    # ------------------------------------------------------------ GPU calls
    def gpu_topk(self, qidx, ctx_lens) -> torch.Tensor:
        wl = self.wl
        out = torch.empty((wl.batch, wl.queries, wl.topk), dtype=torch.int32, device=self.dev)
        self.ctx.index_topk(self.to_dev(qidx), self.w, self.to_dev(ctx_lens), out)
        return out

    def gpu_resolve(self, topk: torch.Tensor, ctx_lens):
        wl = self.wl
        rows = torch.empty_like(topk)
        stats = torch.empty((wl.batch, 4), dtype=torch.int32, device=self.dev)
        self.ctx.resolve(topk, self.to_dev(ctx_lens), rows, stats)
        return rows, stats

    def gpu_decode(self, layer: int, q, rows: torch.Tensor, ctx_lens):
        wl = self.wl
        out = torch.empty((wl.batch, wl.queries, 64, 512), dtype=torch.bfloat16, device=self.dev)
        lse = torch.empty((wl.batch, wl.queries, 64), dtype=torch.float32, device=self.dev)
        self.ctx.decode(layer, self.to_dev(q), rows, self.to_dev(ctx_lens), self.sm_scale, out, lse)
        return out, lse

    # ------------------------------------------------------------ oracle
    def keys(self, b: int) -> np.ndarray:
        if b not in self._keys:
            L = int(self.wl.ctx[b]) + self.wl.steps * self.wl.queries
            codes, scale = synth.idx_tokens(self.wl, b, 0, L)
            self._keys[b] = oracle.dequant_idx_keys(codes, scale)
        return self._keys[b]

    def oracle_scores(self, b: int, qidx, ctx_len: int):
        return oracle.indexer_scores(qidx[b], self.w_np[b], self.keys(b)[:ctx_len])

    def oracle_topk(self, b: int, qidx, ctx_len: int):
        sc = self.oracle_scores(b, qidx, ctx_len)
        return np.stack([oracle.topk_select(s, self.wl.topk) for s in sc]), sc

    def oracle_resolve(self, b: int, topk_b: np.ndarray, window_start: int | None = None):
        lay = self.lay
        return oracle.resolve(topk_b, lay.block_table[b], lay.host_block_table[b], self.hot[b],
                              self.states[b], self.pool, window_start)

    def oracle_release(self, b: int) -> list:
        return oracle.release_hot(self.states[b], self.hot[b], self.pool)

    def oracle_attention(self, b: int, j: int, layer: int, tokens: np.ndarray, q) -> tuple:
        rows = synth.latent_tokens(self.wl, b, layer, tokens)
        lat = oracle.decode_latent_rows(rows, self.wl.kv_dtype)
        return oracle.attention(q[b, j], lat, self.sm_scale)

    def close(self):
        self.ctx.close()


# ---------------------------------------------------------------- comparisons

def check_topk(gpu: np.ndarray, scores: np.ndarray, K: int) -> int:
    """Assert the GPU top-K of one query is a valid answer; return how many tokens differ from
    the oracle's own choice (all of them inside the tie band)."""
    L = scores.shape[0]
    n = min(K, L)
    assert np.all(gpu[n:] == -1), "padding"
    sel = gpu[:n]
    assert np.all(np.diff(sel) > 0), "ascending and distinct"
    assert sel[0] >= 0 and sel[-1] < L
    ref = oracle.topk_select(scores, K)[:n]
    if np.array_equal(sel, ref):
        return 0
    T = np.sort(scores)[::-1][n - 1]
    band = TIE_REL * abs(T)
    diff = np.setxor1d(sel, ref)
    assert np.all(np.abs(scores[diff] - T) <= band), \
        f"top-K differs outside the tie band: {diff[:8]} scores {scores[diff[:8]]} K-th {T}"
    return len(diff) // 2


def check_attention(out_gpu: np.ndarray, lse_gpu: np.ndarray, out_ref: np.ndarray, lse_ref: np.ndarray):
    err = np.abs(out_gpu - out_ref)
    bound = ATOL + RTOL * np.abs(out_ref)
    assert np.all(err <= bound), f"attention max excess {np.max(err - bound):.3e}"
    rel = np.linalg.norm(out_gpu - out_ref) / max(np.linalg.norm(out_ref), 1e-30)
    assert rel <= REL_L2_MAX, f"relative L2 {rel:.3e}"
    assert np.all(np.abs(lse_gpu - lse_ref) <= 1e-3 + 1e-4 * np.abs(lse_ref)), "lse"
    return rel


def check_content(gw: GpuWorkload, b: int, row_ids: np.ndarray, tokens: np.ndarray):
    """Every resolved row holds the canonical bytes of its token, in every layer."""
    wl = gw.wl
    valid = tokens >= 0
    toks, rids = tokens[valid], row_ids[valid]
    n_rows_pool = gw.lay.num_gpu_blocks * 64
    assert np.all((rids >= 0) & (rids < n_rows_pool))
    kv = gw.ctx.kv_pool.view(wl.n_layers, n_rows_pool, wl.row_bytes)
    idx = torch.from_numpy(rids.astype(np.int64)).to(gw.dev)
    for layer in range(wl.n_layers):
        got = kv[layer].index_select(0, idx).cpu().numpy()
        want = synth.latent_tokens(wl, b, layer, toks)
        assert np.array_equal(got, want), f"content mismatch request {b} layer {layer}"
