"""Pins of the oracle's fused resolver (textbook LRU models, invariants, content)."""
from collections import OrderedDict

import numpy as np
import pytest

import oracle
from oracle.hisparse_oracle import ResolveError

BLOCK = 64


def _tables(n_pages, resident_pages, H, rng):
    bt = np.full(n_pages, -1, np.int32)
    hbt = np.full(n_pages, -1, np.int32)
    ids = rng.permutation(1000).astype(np.int32)
    r = 0
    for p in range(n_pages):
        if p in resident_pages:
            bt[p] = ids[r]
            r += 1
        else:
            hbt[p] = 500 + p
    hot = ids[r:r + H // BLOCK].copy()
    return bt, hbt, hot


def test_single_access_equals_textbook_lru():
    # with one selected token per call the (stamp, slot) rule is the classic LRU
    # cache: a hit moves to the back, a miss evicts the front (empty slots first).
    rng = np.random.default_rng(0)
    H, n_pages = 128, 8
    bt, hbt, hot = _tables(n_pages, set(), H, rng)
    st = oracle.HotState.cold(H, n_pages * BLOCK)
    lru = OrderedDict((s, None) for s in range(H))             # slot -> token, front = LRU
    where = {}
    for call in range(3000):
        t = int(rng.integers(0, 200))                          # > H distinct tokens: evictions
        row_ids, copies, stats = oracle.resolve(np.array([[t]]), bt, hbt, hot, st)
        if t in where:
            s = where[t]
            lru.move_to_end(s)
            assert stats[1:3] == (1, 0)
        else:
            s, old = next(iter(lru.items()))
            if old is not None:
                del where[old]
            lru[s] = t
            lru.move_to_end(s)
            where[t] = s
            assert stats[1:3] == (0, 1) and copies[0][1] == s
        assert row_ids[0, 0] == hot[s // BLOCK] * BLOCK + s % BLOCK


def _ordered_list_model(calls, H, resident):
    """Recency list of slots; every slot touched in one call is used 'at the same time'
    and ranks after untouched slots, ties by slot index.  Per call: the slot contents and the
    counts (resident tokens, hot hits, misses, 64-slot pages holding a token) counted here by
    hand from the model's own state."""
    order = list(range(H))
    slot_token = [-1] * H
    where = {}
    out = []
    for U in calls:
        U = sorted(set(U))
        n_res = sum(1 for t in U if t in resident)
        hits = {where[t] for t in U if t not in resident and t in where}
        misses = [t for t in U if t not in resident and t not in where]
        free = [s for s in order if s not in hits]
        victims = free[:len(misses)]
        for t, s in zip(misses, victims):
            if slot_token[s] != -1:
                del where[slot_token[s]]
            slot_token[s] = t
            where[t] = s
        touched = hits | set(victims)
        order = [s for s in order if s not in touched] + sorted(touched)
        # pages of the hot buffer in use: a page counts once any of its 64 slots holds a token
        pages_in_use = len({s // BLOCK for s in range(H) if slot_token[s] != -1})
        out.append((list(slot_token), (n_res, len(hits), len(misses), pages_in_use)))
    return out


@pytest.mark.parametrize("H", [64, 128, 192])
def test_multi_token_calls_match_ordered_list_model(H):
    rng = np.random.default_rng(H)
    n_pages = 12
    resident_pages = {10, 11}
    bt, hbt, hot = _tables(n_pages, resident_pages, H, rng)
    resident = {t for p in resident_pages for t in range(p * BLOCK, (p + 1) * BLOCK)}
    st = oracle.HotState.cold(H, n_pages * BLOCK)
    calls = []
    for _ in range(60):
        n = int(rng.integers(1, H // 2))
        calls.append(list(rng.choice(n_pages * BLOCK, n, replace=False)))
    model = _ordered_list_model(calls, H, resident)
    partial_pages = 0
    for U, (expect, counts) in zip(calls, model):
        S = 2
        topk = np.full((S, len(U)), -1, np.int32)
        half = len(U) // 2
        topk[0, :len(U) - half] = np.sort(U[half:])
        topk[1, :half] = np.sort(U[:half])
        _, _, stats = oracle.resolve(topk, bt, hbt, hot, st)
        assert list(st.slot_token) == expect
        assert stats == counts
        partial_pages += int(sum(s != -1 for s in expect) % BLOCK != 0)
    assert partial_pages > 0  # some calls leave a hot page partly filled


def test_invariants_over_steps_and_content():
    rng = np.random.default_rng(7)
    H, n_pages, S, K = 256, 16, 2, 48
    bt, hbt, hot = _tables(n_pages, {14, 15}, H, rng)
    st = oracle.HotState.cold(H, n_pages * BLOCK)
    # canonical content of token t is t itself; a toy KV pool of row ids
    kv = np.full(1000 * BLOCK, -7, np.int64)
    for p in (14, 15):
        kv[bt[p] * BLOCK:(bt[p] + 1) * BLOCK] = np.arange(p * BLOCK, (p + 1) * BLOCK)
    host = np.arange(n_pages * BLOCK)                          # host row of page p at 500+p
    prev = None
    for step in range(40):
        if step % 7 == 3 and prev is not None:
            topk = prev.copy()
        else:
            topk = np.stack([np.sort(rng.choice(n_pages * BLOCK, K, replace=False)) for _ in range(S)])
            topk = topk.astype(np.int32)
        cold_before = st.step == 0
        before = st.copy()
        row_ids, copies, stats = oracle.resolve(topk, bt, hbt, hot, st)
        U = np.unique(topk)
        non_res = [t for t in U if bt[t // BLOCK] < 0]
        # counts by hand: resident union tokens (pages 14 and 15), hits, misses, and the hot
        # pages holding at least one token
        assert stats[0] == sum(1 for t in U if t // BLOCK in (14, 15))
        assert stats[1] == sum(1 for t in non_res if before.tok2slot[t] != -1)
        assert stats[2] == len(copies) == len(non_res) - stats[1]
        filled = [s for s in range(H) if st.slot_token[s] != -1]
        assert stats[3] == len({s // BLOCK for s in filled})
        if cold_before:
            assert stats[2] == len(non_res) and stats[1] == 0
        if prev is not None and np.array_equal(prev, topk):
            assert stats[2] == 0                                 # identical call: no misses
        hit_slots = {int(before.tok2slot[t]) for t in non_res if before.tok2slot[t] != -1}
        assert not hit_slots & {c[1] for c in copies}           # never evict a hit
        for t, s, hrow, dst in copies:
            assert hrow == (500 + t // BLOCK) * BLOCK + t % BLOCK
            kv[dst] = host[t]                                   # the single-row copy
        # tok2slot and slot_token are inverse maps; resident tokens never hot
        for s in range(H):
            if st.slot_token[s] != -1:
                assert st.tok2slot[st.slot_token[s]] == s
                assert bt[st.slot_token[s] // BLOCK] < 0
        assert (st.tok2slot != -1).sum() == (st.slot_token != -1).sum()
        # content: every row id holds its token's canonical row
        for j in range(S):
            for k in range(K):
                assert kv[row_ids[j, k]] == topk[j, k]
        prev = topk
    assert st.step == 40


def test_capacity_rule_and_errors():
    rng = np.random.default_rng(8)
    H = 64
    bt, hbt, hot = _tables(4, set(), H, rng)
    st = oracle.HotState.cold(H, 4 * BLOCK)
    oracle.resolve(np.arange(64, dtype=np.int32)[None], bt, hbt, hot, st)     # S*K = H fits
    with pytest.raises(ResolveError):
        oracle.resolve(np.arange(64, 129, dtype=np.int32)[None], bt, hbt, hot, st)
    hbt2 = hbt.copy()
    hbt2[2] = -1
    st2 = oracle.HotState.cold(H, 4 * BLOCK)
    with pytest.raises(ResolveError):
        oracle.resolve(np.array([[130]], np.int32), bt, hbt2, hot, st2)
