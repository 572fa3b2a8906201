"""Algorithmic bytes and FLOPs of the decode step (what a roofline is priced on).

Per-unit figures follow Part 2, footnote 1 (sparse MLA) and footnote 3
(per-token KV footprint) of the GLM-5.3 pages:

* a selected FP8 row costs its 656 stored bytes plus a 4-byte index;
* each head adds 2,176 bytes of bf16 query and output (576 + 512 values);
* each (head, row) pair costs 2,176 FLOPs: a multiply-add over 576 dims for
  QK and over 512 dims for PV;
* an FP8 indexer key is 128 one-byte values plus a 4-byte scale (132 bytes).

The indexer figures are this build's own (not printed on the pages): scoring
one key for one query costs 32 heads x 128 dims x 2 FLOPs; its bytes are the
keys streamed once plus the queries, weights and the top-K list written.
"""
from __future__ import annotations

ROW_BYTES = {0: 1152, 1: 656}          # bf16 / FP8 latent row
IDX_KEY_BYTES = {0: 256, 1: 132}       # bf16 / FP8 indexer key per token
ROW_INDEX_BYTES = 4
HEAD_IO_BYTES = (576 + 512) * 2        # bf16 query in, bf16 output out, per head
FLOPS_PER_HEAD_ROW = 2 * 576 + 2 * 512
N_HEADS = 64
IDX_HEADS, IDX_DIM = 32, 128
IDX_FLOPS_PER_KEY = IDX_HEADS * IDX_DIM * 2
IDX_QUERY_BYTES = IDX_HEADS * IDX_DIM * 2 + IDX_HEADS * 4   # bf16 q + fp32 weights


def sparse_mla_bytes(n_rows: int, n_heads: int = N_HEADS, kv_dtype: int = 1) -> int:
    """Bytes one query moves in sparse MLA: gathered rows + index, query and output."""
    return n_rows * (ROW_BYTES[kv_dtype] + ROW_INDEX_BYTES) + n_heads * HEAD_IO_BYTES


def sparse_mla_flops(n_rows: int, n_heads: int = N_HEADS) -> int:
    return n_heads * n_rows * FLOPS_PER_HEAD_ROW


def indexer_bytes(ctx: int, S: int, K: int, idx_dtype: int = 1) -> int:
    """One request: every key streamed once, S queries + weights in, S top-K lists out."""
    return ctx * IDX_KEY_BYTES[idx_dtype] + S * IDX_QUERY_BYTES + S * K * 4


def sweep_bytes(ctx: int, S: int, idx_dtype: int = 1) -> int:
    """One request, score sweep only: every key streamed once, S queries + weights in (the
    scores it hands to the select are an intermediate, not counted)."""
    return ctx * IDX_KEY_BYTES[idx_dtype] + S * IDX_QUERY_BYTES


def indexer_flops(ctx: int, S: int) -> int:
    """One request: each of the S queries scores the rows it sees."""
    return sum((ctx - S + 1 + j) * IDX_FLOPS_PER_KEY for j in range(S))


def kv_bytes_per_token(mla_layers: int = 78, idx_layers: int = 21, mtp_bytes: int = 788,
                       kv_dtype: int = 1) -> int:
    """Per-token KV footprint of a model (footnote 3 counts GLM-5.3 this way)."""
    return mla_layers * ROW_BYTES[kv_dtype] + idx_layers * IDX_KEY_BYTES[1] + mtp_bytes


def step_work(ctx_lens, S: int, K: int, n_layers: int, kv_dtype: int, idx_dtype: int) -> dict:
    """Algorithmic work of one decode step of a batch (ctx_lens = rows present per request)."""
    idx_b = idx_f = gat_b = att_f = 0
    for L in ctx_lens:
        L = int(L)
        idx_b += indexer_bytes(L, S, K, idx_dtype)
        idx_f += indexer_flops(L, S)
        for j in range(S):
            n = min(K, L - S + 1 + j)
            gat_b += n_layers * sparse_mla_bytes(n, kv_dtype=kv_dtype)
            att_f += n_layers * sparse_mla_flops(n)
    return {"indexer_bytes": idx_b, "indexer_flops": idx_f, "gather_bytes": gat_b,
            "attention_flops": att_f}
