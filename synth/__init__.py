"""Seeded synthetic workloads for the Hybrid HiSparse sparse-MLA decode step.

This package builds the inputs that both the CPU oracle and the GPU path
read: indexer queries and keys, head weights, MLA queries, latent rows, and
the paged layout (block tables, residency, host pool, hot buffer blocks).
It contains none of the method's arithmetic.

Workload shapes follow the pages: 64 MLA heads over a 576-dim latent (512
"nope" + 64 rope) with the value taken as the first 512 dims, FP8 latent rows
of 656 bytes and FP8 indexer keys of 132 bytes per token (GLM-5.3 part-2 page,
footnotes 1 and 3), top-K = 2,048 (part-2 page, "Why not TP or DP?"), a hot
buffer of 2 x top-K rows per request, or (speculative tokens + 2) x top-K
with MTP (Hybrid HiSparse page, "Composing with the rest of vLLM" and the
calculator note).  The value distributions are not on the pages; the recipe
is: keys, latents and MLA queries N(0, 1); head weights U(0, 1); indexer
queries follow q_{n+1} = 0.95 q_n + 0.31 eps per request; 2 % of tokens get
+3 on every key component (a persistent salient set).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

BLOCK = 64
SEED_BASE = 20261202
KIND_W = 6
KIND_UNIFORM = 8


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        u32, i32, i64, f32, f64 = (ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_float, ctypes.c_double)
        L.synth_philox.argtypes = [u32, u32, u32, u32, u32, u32, P]
        L.synth_normals.argtypes = [u32, u32, u32, u32, u32, i32, P]
        L.synth_uniforms.argtypes = [u32, u32, u32, u32, u32, i32, P]
        L.synth_salient_mask.argtypes = [u32, i32, i64, i64, f64, P]
        L.synth_idx_pages.argtypes = [u32, i32, i32, i64, P, P, P, f64, f32]
        L.synth_idx_tokens.argtypes = [u32, i32, i32, i64, i64, P, P, f64, f32]
        L.synth_latent_pages.argtypes = [u32, i32, i32, i32, i64, P, P, P]
        L.synth_latent_tokens.argtypes = [u32, i32, i32, i32, i64, P, P]
        L.synth_qidx_chain.argtypes = [u32, i32, i32, f32, f32, P]
        L.synth_mla_q.argtypes = [u32, i32, i32, i32, P]
        L.synth_encode_bf16.argtypes = [P, i64, P]
        L.synth_encode_e4m3.argtypes = [P, i64, P]
        L.synth_bf16_from_f32.argtypes = [f32]
        L.synth_bf16_from_f32.restype = ctypes.c_uint16
        L.synth_e4m3_from_f32.argtypes = [f32]
        L.synth_e4m3_from_f32.restype = ctypes.c_uint8
        L.synth_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ----------------------------------------------------------------- encoders

def encode_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().synth_encode_bf16(_p(x), x.size, _p(out))
    return out


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().synth_encode_e4m3(_p(x), x.size, _p(out))
    return out


def uniforms(seed: int, kind: int, a: int, b: int, c: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniforms(seed, kind, a, b, c, n, _p(out))
    return out


def normals(seed: int, kind: int, a: int, b: int, c: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normals(seed, kind, a, b, c, n, _p(out))
    return out


# ----------------------------------------------------------------- workloads

RES_FULL, RES_HYBRID, RES_PREFIX = 0, 1, 2


@dataclass
class Workload:
    """One synthetic decode workload (a row of the configuration table)."""

    name: str
    seed: int
    batch: int
    queries: int                 # S: query tokens per request (1, or 4 under MTP3)
    n_layers: int                # sparse-MLA layers sharing one top-K
    ctx: list                    # L_b at step 0 (rows present incl. the S query rows)
    kv_dtype: int                # 0 bf16 rows (1152 B), 1 fp8 rows (656 B)
    idx_dtype: int               # 0 bf16 keys (256 B), 1 fp8 keys + scale (132 B)
    residency: list              # per request: (kind, fraction)
    hot_rows: int
    steps: int
    topk: int = 2048
    drift: tuple = (0.95, 0.31)
    salient_frac: float = 0.02
    salient_shift: float = 3.0
    extra: dict = field(default_factory=dict)

    @property
    def row_bytes(self) -> int:
        return 1152 if self.kv_dtype == 0 else 656

    @property
    def idx_block_bytes(self) -> int:
        return 16384 if self.idx_dtype == 0 else 8448

    @property
    def idx_token_bytes(self) -> int:
        return 256 if self.idx_dtype == 0 else 132

    def ctx_at(self, step: int) -> np.ndarray:
        return np.asarray(self.ctx, np.int64) + step * self.queries

    @property
    def max_ctx(self) -> int:
        return int(max(self.ctx)) + self.steps * self.queries

    @property
    def max_pages(self) -> int:
        return -(-self.max_ctx // BLOCK)


def _loguniform_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    u = uniforms(seed, KIND_UNIFORM, 5, 0, 0, n)
    return [int(math.floor(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]


def _residency_draw(seed: int, n: int) -> list:
    u = uniforms(seed, KIND_UNIFORM, 6, 0, 0, n)
    kinds = [min(2, int(math.floor(3.0 * x))) for x in u]
    return [(RES_FULL, 1.0) if k == 0 else (RES_HYBRID, 0.25) if k == 1 else (RES_PREFIX, 0.0)
            for k in kinds]


def config(index: int, scale: int = 1, steps: int | None = None, batch: int | None = None) -> Workload:
    """The five workloads; `scale` divides every context length (reduced runs)."""
    seed = SEED_BASE + index
    if index == 1:
        B = batch or 1
        return Workload("ctx8k_b1_bf16", seed, B, 1, 1, [8192 // scale] * B, 0, 0,
                        [(RES_FULL, 1.0)] * B, 4096, steps or 1, drift=(1.0, 0.0),
                        salient_frac=0.0)
    if index == 2:
        B = batch or 32
        return Workload("ctx64k_b32_fp8", seed, B, 1, 1, [65536 // scale] * B, 1, 1,
                        [(RES_HYBRID, 0.25)] * B, 4096, steps or 16)
    if index == 3:
        B = batch or 64
        return Workload("ctx128k_b64_mtp3_fp8", seed, B, 4, 1, [131072 // scale] * B, 1, 1,
                        [(RES_HYBRID, 0.10)] * B, 10240, steps or 16)
    if index == 4:
        B = batch or 1
        return Workload("ctx1m_b1_fp8", seed, B, 1, 1, [1048576 // scale] * B, 1, 1,
                        [(RES_PREFIX, 0.0)] * B, 4096, steps or 64)
    if index == 5:
        B = batch or 128
        lens = _loguniform_lengths(seed, B, max(64, 4096 // scale), 1048576 // scale)
        return Workload("mixed_b128_indexshare4_fp8", seed, B, 1, 4, lens, 1, 1,
                        _residency_draw(seed, B), 4096, steps or 32)
    raise ValueError(index)


def toy(seed: int = 7, batch: int = 2, queries: int = 1, ctx=(700, 1333), topk: int = 16,
        hot_rows: int | None = None, n_layers: int = 1, kv_dtype: int = 1, idx_dtype: int = 1,
        residency=None, steps: int = 3, salient_frac: float = 0.02) -> Workload:
    """Small ragged workloads for tests (contexts not multiples of 64)."""
    ctx = list(ctx)[:batch] + [ctx[-1]] * max(0, batch - len(ctx))
    residency = residency or [(RES_HYBRID, 0.25)] * batch
    if hot_rows is None:
        hot_rows = -(-((queries + 1) * topk) // BLOCK) * BLOCK
    return Workload(f"toy{seed}", seed, batch, queries, n_layers, ctx, kv_dtype, idx_dtype,
                    list(residency), hot_rows, steps, topk=topk, salient_frac=salient_frac)


# ----------------------------------------------------------------- layout

@dataclass
class Layout:
    """Block tables and pool sizes of a workload (integers only)."""

    block_table: np.ndarray       # [B][max_pages] int32 GPU block or -1 (placeholder)
    host_block_table: np.ndarray  # [B][max_pages] int32 host block or -1
    idx_block_table: np.ndarray   # [B][max_pages] int32 indexer block
    hot_blocks: np.ndarray        # [B][hot_rows/64] int32 GPU blocks leased for hot rows
    num_gpu_blocks: int
    num_host_blocks: int
    num_idx_blocks: int


def make_layout(wl: Workload) -> Layout:
    """Residency per request at step 0 and seeded block numbering.

    Pages are 64 tokens.  With n = ceil(L/64) pages present, the newest
    ceil(f * n) pages are GPU-resident (at least the tail page, which is never
    evicted); older pages are placeholders whose rows live in the host pool.
    Pages for the tokens of later steps are allocated resident up front.
    Block ids in each pool are a seeded permutation, so requests interleave.
    """
    B, P = wl.batch, wl.max_pages
    hot_pages = wl.hot_rows // BLOCK
    resident = np.zeros((B, P), bool)
    present = np.zeros((B, P), bool)
    for b in range(B):
        n_now = -(-int(wl.ctx[b]) // BLOCK)
        n_all = -(-(int(wl.ctx[b]) + wl.steps * wl.queries) // BLOCK)
        kind, frac = wl.residency[b]
        if kind == RES_FULL:
            n_res = n_now
        elif kind == RES_HYBRID:
            n_res = max(1, math.ceil(frac * n_now))
        else:
            n_res = 1
        present[b, :n_all] = True
        resident[b, n_now - n_res:n_all] = True
    rng = np.random.default_rng(wl.seed)
    n_gpu = int(resident.sum()) + B * hot_pages
    gpu_ids = rng.permutation(n_gpu).astype(np.int32)
    host_mask = present & ~resident
    n_host = int(host_mask.sum())
    host_ids = rng.permutation(max(n_host, 1)).astype(np.int32)[:n_host]
    n_idx = int(present.sum())
    idx_ids = rng.permutation(n_idx).astype(np.int32)

    bt = np.full((B, P), -1, np.int32)
    hbt = np.full((B, P), -1, np.int32)
    ibt = np.full((B, P), -1, np.int32)
    hot = np.zeros((B, max(hot_pages, 1)), np.int32)[:, :hot_pages]
    bt[resident] = gpu_ids[: int(resident.sum())]
    hot[:] = gpu_ids[int(resident.sum()):].reshape(B, hot_pages)
    hbt[host_mask] = host_ids
    ibt[present] = idx_ids
    return Layout(bt, hbt, ibt, np.ascontiguousarray(hot), n_gpu, n_host, n_idx)


# ----------------------------------------------------------------- fills

def fill_idx_pool(wl: Workload, lay: Layout, pool: np.ndarray) -> None:
    """Write every present page's indexer keys into `pool` (uint8, blocks x block bytes)."""
    assert pool.dtype == np.uint8 and pool.size >= lay.num_idx_blocks * wl.idx_block_bytes
    for b in range(wl.batch):
        pages = np.nonzero(lay.idx_block_table[b] >= 0)[0].astype(np.int32)
        dst = lay.idx_block_table[b][pages].astype(np.int64)
        lib().synth_idx_pages(wl.seed, wl.idx_dtype, b, len(pages), _p(pages), _p(dst), _p(pool),
                              wl.salient_frac, wl.salient_shift)


def fill_kv(wl: Workload, lay: Layout, gpu_rows: np.ndarray | None, host_rows: np.ndarray | None,
            layers=None) -> None:
    """Write latent rows: resident pages into `gpu_rows` ([layers][gpu blocks*64] rows), host-only
    pages into `host_rows` ([layers][host blocks*64] rows); both uint8, row_bytes per row."""
    rb = wl.row_bytes
    layers = range(wl.n_layers) if layers is None else layers
    for li, layer in enumerate(layers):
        for b in range(wl.batch):
            for table, buf, nblk in ((lay.block_table, gpu_rows, lay.num_gpu_blocks),
                                     (lay.host_block_table, host_rows, lay.num_host_blocks)):
                if buf is None:
                    continue
                pages = np.nonzero(table[b] >= 0)[0].astype(np.int32)
                if len(pages) == 0:
                    continue
                base = li * nblk * BLOCK
                row0 = (table[b][pages].astype(np.int64) * BLOCK + base)
                assert buf.dtype == np.uint8 and buf.size >= (base + nblk * BLOCK) * rb
                lib().synth_latent_pages(wl.seed, wl.kv_dtype, b, layer, len(pages), _p(pages),
                                         _p(row0), _p(buf))


def idx_tokens(wl: Workload, b: int, t0: int, n: int):
    """Stored indexer keys of tokens [t0, t0+n) of request b in token order.
    bf16: (uint16 [n][128], None); fp8: (uint8 [n][128], float32 [n])."""
    if wl.idx_dtype == 0:
        codes = np.empty((n, 128), np.uint16)
        lib().synth_idx_tokens(wl.seed, 0, b, t0, n, _p(codes), None, wl.salient_frac,
                               wl.salient_shift)
        return codes, None
    codes = np.empty((n, 128), np.uint8)
    scale = np.empty(n, np.float32)
    lib().synth_idx_tokens(wl.seed, 1, b, t0, n, _p(codes), _p(scale), wl.salient_frac,
                           wl.salient_shift)
    return codes, scale


def latent_tokens(wl: Workload, b: int, layer: int, tokens) -> np.ndarray:
    """Stored latent rows (uint8 [n][row_bytes]) of the given tokens of (b, layer)."""
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    out = np.empty((len(tokens), wl.row_bytes), np.uint8)
    lib().synth_latent_tokens(wl.seed, wl.kv_dtype, b, layer, len(tokens), _p(tokens), _p(out))
    return out


def qidx(wl: Workload, b: int, n_query_tokens: int) -> np.ndarray:
    """Indexer queries (bf16 codes [n][32][128]) of request b over flattened query tokens."""
    out = np.empty((n_query_tokens, 32, 128), np.uint16)
    rho, sigma = wl.drift
    lib().synth_qidx_chain(wl.seed, b, n_query_tokens, rho, sigma, _p(out))
    return out


def qidx_step(wl: Workload, step: int, chains=None) -> np.ndarray:
    """[B][S][32][128] bf16 codes of one decode step (query token n = step*S + j)."""
    S = wl.queries
    out = np.empty((wl.batch, S, 32, 128), np.uint16)
    for b in range(wl.batch):
        ch = chains[b] if chains is not None else qidx(wl, b, (step + 1) * S)
        out[b] = ch[step * S:(step + 1) * S]
    return out


def head_weights(wl: Workload) -> np.ndarray:
    """[B][S][32] float32 indexer head weights ~ U(0,1), fixed across steps."""
    w = np.empty((wl.batch, wl.queries, 32), np.float32)
    for b in range(wl.batch):
        for j in range(wl.queries):
            w[b, j] = uniforms(wl.seed, KIND_W, b, j, 0, 32).astype(np.float32)
    return w


def mla_q(wl: Workload, step: int, batches=None) -> np.ndarray:
    """[B][S][64][576] bf16 codes of the MLA queries of one step (fresh N(0,1))."""
    S = wl.queries
    bs = range(wl.batch) if batches is None else batches
    out = np.empty((len(bs), S, 64, 576), np.uint16)
    for i, b in enumerate(bs):
        lib().synth_mla_q(wl.seed, b, step * S, S, _p(out[i]))
    return out


# Prefill inputs of request b: its P new tokens are query tokens numbered from PREFILL_QUERY0 on,
# a range no decode step reaches, so they never repeat a decode step's draws.
PREFILL_QUERY0 = 1 << 24


def prefill_qidx(wl: Workload, b: int, P: int) -> np.ndarray:
    """[P][32][128] bf16 codes: indexer queries of the P new tokens (the request's drifting
    chain: neighbouring prompt tokens are correlated)."""
    return qidx(wl, b, P)


def prefill_head_weights(wl: Workload, b: int, P: int) -> np.ndarray:
    """[P][32] float32 head weights ~ U(0,1), one set per new token."""
    w = np.empty((P, 32), np.float32)
    for i in range(P):
        w[i] = uniforms(wl.seed, KIND_W, b, i, 1, 32).astype(np.float32)
    return w


def prefill_mla_q(wl: Workload, b: int, P: int) -> np.ndarray:
    """[P][64][576] bf16 codes: MLA queries of the P new tokens (fresh N(0,1))."""
    return prefill_mla_q_range(wl, b, 0, P)


def prefill_mla_q_range(wl: Workload, b: int, i0: int, n: int) -> np.ndarray:
    """MLA queries of new tokens i0 .. i0 + n of a prefill (token i's draw does not depend on P)."""
    out = np.empty((n, 64, 576), np.uint16)
    lib().synth_mla_q(wl.seed, b, PREFILL_QUERY0 + i0, n, _p(out))
    return out


def salient_mask(wl: Workload, b: int, t0: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().synth_salient_mask(wl.seed, b, t0, n, wl.salient_frac, _p(out))
    return out.astype(bool)
