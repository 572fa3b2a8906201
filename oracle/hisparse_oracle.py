"""Plain float64 definitions of each stage of the sparse-MLA decode step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  No blocking, fusion
or reordering beyond what each definition states; library primitives used as
single steps: matrix products (``np.matmul``), sorting (``np.lexsort``).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 64  # tokens per page (the workloads' block size)


# ----------------------------------------------------------------- formats

def _e4m3_value(code: int) -> float:
    """OCP 8-bit floating point E4M3 ("FN" variant): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits, subnormals at exponent field 0, no
    infinities, S.1111.111 is NaN.  The pages' FP8 KV and FP8 indexer keys
    are this format (Part 2, footnotes 1 and 3)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact float64 values of E4M3 codes."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bf16 is the upper half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_idx_keys(codes: np.ndarray, scale) -> np.ndarray:
    """Indexer keys as real numbers, [L][128] float64.

    bf16 keys (``scale is None``) decode directly.  FP8 keys are 128 E4M3
    values with one fp32 scale per token, 132 bytes per token (Part 2,
    footnote 3); the key is code * scale, exact in float64.
    """
    if scale is None:
        return bf16_decode(codes)
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


def decode_latent_rows(rows: np.ndarray, kv_dtype: int) -> np.ndarray:
    """Stored latent rows -> [n][576] float64 (512 "nope" dims, then 64 rope).

    kv_dtype 0: 576 bf16 values (1152 bytes).
    kv_dtype 1: the 656-byte FP8 row of Part 2, footnote 1.  The pages give
    only its size; the reading taken: bytes [0,512) E4M3 nope codes, [512,640)
    64 bf16 rope values, [640,644) the fp32 scale of the nope codes, rest zero.
    """
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    if kv_dtype == 0:
        return bf16_decode(rows.view(np.uint16).reshape(n, 576))
    nope = e4m3_decode(rows[:, :512])
    rope = bf16_decode(rows[:, 512:640].copy().view(np.uint16))
    scale = rows[:, 640:644].copy().view(np.float32).astype(np.float64)
    return np.concatenate([nope * scale, rope], axis=1)


# ----------------------------------------------------------------- indexer

def indexer_scores(q_idx_bits: np.ndarray, w: np.ndarray, keys: np.ndarray) -> list:
    """Indexer scores of one request (Part 1, "Using sparsity when it is
    needed": the indexer picks the top-K tokens; Part 2, "Why not TP or DP?":
    it scores every earlier token).

    The formula is not on the pages; the reading taken is
        s_j(t) = sum_h w[j,h] * max(0, sum_d q[j,h,d] * k[t,d])
    with 32 heads of 128 dims and one 128-dim key per token.

    q_idx_bits  [S][32][128] bf16 codes of the S query tokens
    w           [S][32] float32 head weights
    keys        [L][128] float64 keys of the L rows present (the S query
                tokens' own rows are the last S)
    Returns S arrays; query j sees rows t < L - S + 1 + j (its own row and
    every earlier one, never a later draft token).  -0 is returned as +0.
    """
    S = q_idx_bits.shape[0]
    L = keys.shape[0]
    q = bf16_decode(q_idx_bits).reshape(S, 32, 128)
    out = []
    for j in range(S):
        Lj = L - S + 1 + j
        dots = np.matmul(q[j], keys[:Lj].T)              # [32][Lj]
        relu = np.maximum(dots, 0.0)
        s = np.matmul(w[j].astype(np.float64), relu)     # [Lj]
        out.append(s + 0.0)
    return out


def topk_select(scores: np.ndarray, K: int) -> np.ndarray:
    """Top-K of one query (K = 2,048 on the pages).

    The K = min(K, L_j) tokens ranked first by (score descending, token index
    ascending); ties go to the lower index.  Returned in ascending token
    order, padded with -1 to K.  With L_j <= K every token is selected, the
    case that keeps short prompts on the sparse kernel (Part 2, "Try it").
    """
    L = scores.shape[0]
    order = np.lexsort((np.arange(L), -np.asarray(scores, dtype=np.float64)))
    sel = np.sort(order[: min(K, L)])
    out = np.full(K, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


# ----------------------------------------------------------------- resolver

@dataclass
class HotState:
    """Hot buffer of one request: H token-indexed slots (Part 1, "Using
    sparsity when it is needed": hot pages are indexed by token)."""

    slot_token: np.ndarray   # [H] int32, -1 empty
    slot_stamp: np.ndarray   # [H] int32, -1 never used
    tok2slot: np.ndarray     # [L_max] int32, -1 absent
    step: int = 0            # resolve calls made so far

    @staticmethod
    def cold(H: int, L_max: int) -> "HotState":
        return HotState(np.full(H, -1, np.int32), np.full(H, -1, np.int32),
                        np.full(L_max, -1, np.int32), 0)

    def copy(self) -> "HotState":
        return HotState(self.slot_token.copy(), self.slot_stamp.copy(), self.tok2slot.copy(),
                        self.step)


class ResolveError(RuntimeError):
    pass


class HotPool:
    """The shared pool that hot pages are leased from (Part 1, "How it works": hot-buffer pages
    are ordinary KV blocks leased from the same pool as resident pages, taken when a request
    first needs them and given back when it no longer does; one request's freed blocks become
    another's hot capacity).

    Reading taken (the pages give no order): a first-in first-out list of free GPU blocks.  A
    lease takes the block at the front; a returned block goes to the back."""

    def __init__(self, blocks=()):
        self.free = [int(x) for x in blocks]

    def give_back(self, blocks) -> None:
        self.free.extend(int(x) for x in blocks)

    def lease(self) -> int:
        if not self.free:
            raise ResolveError("no free block left in the hot pool")
        return self.free.pop(0)


def resolve(topk: np.ndarray, block_table: np.ndarray, host_block_table: np.ndarray,
            hot_blocks: np.ndarray, st: HotState, pool: HotPool | None = None,
            window_start: int | None = None):
    """Fused top-K resolver of one request, one call (Part 1, "How it works":
    a resident token is read where it is, a hot token is read and its LRU
    entry refreshed, a miss copies its single row from pinned host memory into
    an LRU slot; the resolver hands out HMA row ids, gathered with one stride).

    topk              [S][K] int32, ascending, -1 padded (one list per query)
    block_table       [pages] int32, GPU block or -1 (placeholder)
    host_block_table  [pages] int32, host block or -1
    hot_blocks        [H/64] int32, GPU blocks holding the hot slots; with a `pool`, -1 marks a
                      hot page not leased yet, and leases are written into it in place
    st                hot state, updated in place
    pool              the shared pool hot pages are leased from, or None when every hot page
                      has its block from the start
    window_start      the call counter at which the request's current plan window began (None:
                      this call begins one).  Part 1, "Composing with the rest of vLLM":
                      speculative decoding runs on per-step plans that can be replayed and share
                      the request's hot state.  Reading taken: a plan is the row ids one call
                      emits; no slot touched by a call of the current window is given to a miss,
                      so every plan of the window keeps reading its rows until a later call
                      begins a new window (for instance once drafts are rejected).

    Readings taken where the pages are silent:
      * the LRU clock is the call counter; a hit and a fill both stamp it;
      * resident pages take precedence and never touch the LRU;
      * victims are the slots not touched in this window (this call, when it
        begins one), in (stamp, slot) order, empty slots (stamp -1) first; the
        i-th miss in ascending token order takes the i-th victim;
      * a miss whose victim slot lies on a hot page without a block leases one
        from the pool (empty slots fill in ascending order, so pages are leased
        in ascending order, as the request first needs them);
      * a placeholder page without a host copy is an error.
    Returns (row_ids [S][K] int32, copies, stats) where copies lists
    (token, slot, host_row, dst_row) and stats = (resident, hit, miss, pages
    of hot slots in use).
    """
    step = st.step
    protect = step if window_start is None else int(window_start)
    U = np.unique(topk[topk >= 0])                                   # sorted union
    page = U // BLOCK
    resident = block_table[page] >= 0
    hot = ~resident & (st.tok2slot[U] != -1)
    miss = ~resident & ~hot

    for t in U[hot]:                                                 # refresh hits
        st.slot_stamp[st.tok2slot[t]] = step

    cand = np.nonzero(st.slot_stamp < protect)[0]                    # untouched in the window
    cand = cand[np.lexsort((cand, st.slot_stamp[cand]))]             # (stamp, slot) order
    misses = U[miss]
    if misses.shape[0] > cand.shape[0]:
        raise ResolveError("hot buffer smaller than the misses of one call")
    copies = []
    for i, t in enumerate(misses):                                   # ascending token order
        s = int(cand[i])
        u = int(st.slot_token[s])
        if u != -1:
            st.tok2slot[u] = -1
        st.slot_token[s] = t
        st.slot_stamp[s] = step
        st.tok2slot[t] = s
        hb = int(host_block_table[t // BLOCK])
        if hb < 0:
            raise ResolveError(f"token {t}: placeholder page without a host copy")
        if hot_blocks[s // BLOCK] < 0:
            if pool is None:
                raise ResolveError(f"hot page {s // BLOCK} has no block")
            hot_blocks[s // BLOCK] = pool.lease()
        dst = int(hot_blocks[s // BLOCK]) * BLOCK + s % BLOCK
        copies.append((int(t), s, hb * BLOCK + int(t) % BLOCK, dst))

    row_of = {}
    for t in U:
        blk = int(block_table[t // BLOCK])
        if blk >= 0:
            row_of[int(t)] = blk * BLOCK + int(t) % BLOCK
        else:
            s = int(st.tok2slot[t])
            row_of[int(t)] = int(hot_blocks[s // BLOCK]) * BLOCK + s % BLOCK
    row_ids = np.full(topk.shape, -1, np.int32)
    for idx in zip(*np.nonzero(topk >= 0)):
        row_ids[idx] = row_of[int(topk[idx])]

    used = int((st.slot_token != -1).sum())
    stats = (int(resident.sum()), int(hot.sum()), int(miss.sum()), -(-used // BLOCK))
    st.step = step + 1
    return row_ids, copies, stats


def release_hot(st: HotState, hot_blocks: np.ndarray, pool: HotPool | None = None) -> list:
    """A request gives up its hot buffer (Part 1, "How it works": hot pages go back to the pool
    when no longer needed; a freed block can become another request's hot capacity).  Its hot
    state becomes cold, as for a new request in that slot; with a pool, its leased blocks go
    back to the pool in page order and its hot-page table is cleared to -1.  Returns the blocks
    given back."""
    back = []
    if pool is not None:
        back = [int(x) for x in hot_blocks if x >= 0]
        pool.give_back(back)
        hot_blocks[:] = -1
    st.slot_token[:] = -1
    st.slot_stamp[:] = -1
    st.tok2slot[:] = -1
    st.step = 0
    return back


# ----------------------------------------------------------------- attention

def attention(q_bits: np.ndarray, latent: np.ndarray, sm_scale: float):
    """Sparse MLA decode attention of one query over its selected rows (Part
    2, "Why not TP or DP?": all 64 heads share one latent row; footnote 1: QK
    runs over 576 dims and PV over 512).  Dense softmax over the selected
    rows; the value is the first 512 dims of the latent row.

    q_bits   [64][576] bf16 codes
    latent   [n][576] float64 rows (n >= 1)
    Returns (out [64][512], lse [64]) in float64.
    """
    q = bf16_decode(q_bits).reshape(64, 576)
    logits = sm_scale * np.matmul(q, latent.T)                        # [64][n]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    l = p.sum(axis=1, keepdims=True)
    out = np.matmul(p, latent[:, :512]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# ------------------------------------------------------- host pool write side

def materialize_pages(gpu_rows: np.ndarray, host_rows: np.ndarray, block_table: np.ndarray,
                      host_block_table: np.ndarray, pages, n_layers: int) -> None:
    """Copy completed pages to host memory (Part 1, "How it works", the paragraph after the
    three residency states: a completed cacheable prefix page is queued for a copy to CPU
    memory while the GPU keeps serving it; all sparse-MLA layers are copied together).

    gpu_rows  [n_layers][gpu blocks * 64][row bytes] uint8 (rows as stored on the GPU)
    host_rows [n_layers][host blocks * 64][row bytes] uint8, written in place
    pages     (request, page) pairs.  A page with no GPU block or no host block is skipped.
    """
    for b, p in pages:
        g, h = int(block_table[b, p]), int(host_block_table[b, p])
        if g < 0 or h < 0:
            continue
        for layer in range(n_layers):
            host_rows[layer, h * BLOCK:(h + 1) * BLOCK] = gpu_rows[layer, g * BLOCK:(g + 1) * BLOCK]


def release_pages(block_table: np.ndarray, host_block_table: np.ndarray, pages, ctx_lens) -> list:
    """A page gives up its GPU block without a second copy (Part 1, "How it works": once its
    host copy exists, the page can release its GPU slot when the pool fills; the tail is never
    evicted).  Returns the freed GPU block per entry (-1 where nothing was given up) and writes
    the placeholder -1 into block_table in place.

    Reading: a page whose host block is missing keeps its GPU block; so do the tail page
    (holding token ctx_len - 1) and pages past it; a page listed twice is given up once.
    """
    freed = []
    for b, p in pages:
        tail = (int(ctx_lens[b]) - 1) // BLOCK
        g, h = int(block_table[b, p]), int(host_block_table[b, p])
        if p >= tail or h < 0 or g < 0:
            freed.append(-1)
            continue
        block_table[b, p] = -1
        freed.append(g)
    return freed
