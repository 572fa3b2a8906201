"""Pins of the oracle's hot-page leasing and plan windows.

Part 1, "How it works": hot-buffer pages are ordinary blocks leased from the same pool as
resident pages, taken when a request first needs them and given back when it no longer does;
one request's freed blocks become another's hot capacity.  Part 1, "Composing with the rest of
vLLM": speculative decoding runs on per-step resolver plans that can be replayed and share the
request's hot state.

The models here are written independently of the oracle's stamp arithmetic: a recency list of
slots per request (as in test_oracle_resolve.py), a plain deque of free blocks, and a set of
slots pinned by the calls of the current window.
"""
from collections import deque

import numpy as np
import pytest

import oracle
from oracle.hisparse_oracle import ResolveError

BLOCK = 64


class LeaseModel:
    """Recency list per request; a slot touched by a call of the current window is pinned and
    never given to a miss; a hot page takes the front block of the free deque the first time a
    token is filled into one of its slots; a released request hands its blocks back, page by
    page, at the back of the deque."""

    def __init__(self, H, free_blocks):
        self.H = H
        self.pool = deque(int(x) for x in free_blocks)
        self.req = {}

    def _r(self, b):
        if b not in self.req:
            self.req[b] = dict(order=list(range(self.H)), slot_token=[-1] * self.H, where={},
                               pages=[-1] * (self.H // BLOCK), pinned=set())
        return self.req[b]

    def call(self, b, U, resident, begin=True):
        r = self._r(b)
        if begin:
            r["pinned"] = set()
        U = sorted(set(int(t) for t in U))
        hits = {r["where"][t] for t in U if t not in resident and t in r["where"]}
        misses = [t for t in U if t not in resident and t not in r["where"]]
        pinned = r["pinned"] | hits
        free = [s for s in r["order"] if s not in pinned]
        if len(misses) > len(free):
            raise ResolveError("model: window holds more rows than the hot buffer")
        victims = free[:len(misses)]
        for t, s in zip(misses, victims):
            old = r["slot_token"][s]
            if old != -1:
                del r["where"][old]
            r["slot_token"][s] = t
            r["where"][t] = s
            if r["pages"][s // BLOCK] == -1:
                if not self.pool:
                    raise ResolveError("model: pool empty")
                r["pages"][s // BLOCK] = self.pool.popleft()
        touched = hits | set(victims)
        r["order"] = [s for s in r["order"] if s not in touched] + sorted(touched)
        r["pinned"] = pinned | set(victims)
        return {t: r["pages"][r["where"][t] // BLOCK] * BLOCK + r["where"][t] % BLOCK
                for t in U if t not in resident}

    def release(self, b):
        r = self._r(b)
        for blk in r["pages"]:
            if blk != -1:
                self.pool.append(blk)
        del self.req[b]


def _tables(n_pages, resident_pages, seed):
    bt = np.full(n_pages, -1, np.int32)
    hbt = np.full(n_pages, -1, np.int32)
    for i, p in enumerate(sorted(resident_pages)):
        bt[p] = 900 + i + 10 * seed
    for p in range(n_pages):
        if p not in resident_pages:
            hbt[p] = 300 + p
    return bt, hbt


def _topk(U, S, rng):
    """Spread the tokens U over S ascending, -1 padded lists (one per query)."""
    U = np.array(sorted(U), np.int32)
    parts = np.array_split(rng.permutation(U), S)
    K = max(len(p) for p in parts) + 2
    out = np.full((S, K), -1, np.int32)
    for j, p in enumerate(parts):
        out[j, :len(p)] = np.sort(p)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_leasing_across_requests_equals_fifo_model(seed):
    rng = np.random.default_rng(100 + seed)
    H, n_pages, B = 192, 10, 3
    resident_pages = {8, 9}
    resident = {t for p in resident_pages for t in range(p * BLOCK, (p + 1) * BLOCK)}
    tables = [_tables(n_pages, resident_pages, b) for b in range(B)]
    initial = list(rng.permutation(np.arange(40, 48)))            # 8 free blocks for 3 x 3 pages
    pool = oracle.HotPool(initial)
    model = LeaseModel(H, initial)
    states = [oracle.HotState.cold(H, n_pages * BLOCK) for _ in range(B)]
    hot = [np.full(H // BLOCK, -1, np.int32) for _ in range(B)]
    leased_seen = 0
    for call in range(120):
        b = int(rng.integers(0, B))
        if len(pool.free) < 3:                                     # a request ends; its slot is reused
            b = max(range(B), key=lambda x: int((hot[x] != -1).sum()))
            back = oracle.release_hot(states[b], hot[b], pool)
            model.release(b)
            assert (hot[b] == -1).all() and states[b].step == 0
            assert back == [x for x in back if x >= 0]
            assert list(pool.free) == list(model.pool)
            continue
        n = int(rng.integers(1, 70))
        U = rng.choice(n_pages * BLOCK, n, replace=False)
        topk = _topk(U, 2, rng)
        expect = model.call(b, U, resident)
        bt, hbt = tables[b]
        before = hot[b].copy()
        rows, copies, stats = oracle.resolve(topk, bt, hbt, hot[b], states[b], pool)
        # the blocks leased in this call, in page order, came off the front of the deque
        new = [int(x) for p, x in enumerate(hot[b]) if before[p] == -1 and x != -1]
        leased_seen += len(new)
        assert [int(x) for x in hot[b]] == model.req[b]["pages"]
        assert list(pool.free) == list(model.pool)
        for j in range(topk.shape[0]):
            for k in range(topk.shape[1]):
                t = int(topk[j, k])
                if t < 0:
                    assert rows[j, k] == -1
                elif t in resident:
                    assert rows[j, k] == bt[t // BLOCK] * BLOCK + t % BLOCK
                else:
                    assert rows[j, k] == expect[t]
        # leased pages are exactly the pages holding a filled slot (empty slots fill in order)
        used = int((states[b].slot_token != -1).sum())
        assert int((hot[b] != -1).sum()) == -(-used // BLOCK) == stats[3]
        # conservation: every block is either free or held by exactly one request
        held = [int(x) for h in hot for x in h if x != -1]
        assert sorted(held + list(pool.free)) == sorted(int(x) for x in initial)
    assert leased_seen > len(initial)                               # freed blocks were reused


def test_leasing_is_invisible_to_the_slot_logic():
    # the same calls with every hot page's block given up front produce the same slots,
    # stamps and row ids as leasing the pages on first need
    rng = np.random.default_rng(7)
    H, n_pages = 256, 12
    bt, hbt = _tables(n_pages, {11}, 0)
    pool = oracle.HotPool([60, 61, 62, 63])
    st_l = oracle.HotState.cold(H, n_pages * BLOCK)
    hot_l = np.full(H // BLOCK, -1, np.int32)
    calls = [_topk(rng.choice(n_pages * BLOCK, int(rng.integers(1, 120)), replace=False), 3, rng)
             for _ in range(30)]
    out_l = [oracle.resolve(tk, bt, hbt, hot_l, st_l, pool)[0] for tk in calls]
    st_s = oracle.HotState.cold(H, n_pages * BLOCK)
    hot_s = hot_l.copy()                                            # the blocks leasing ended with
    out_s = [oracle.resolve(tk, bt, hbt, hot_s, st_s)[0] for tk in calls]
    for a, b in zip(out_l, out_s):
        assert np.array_equal(a, b)
    assert np.array_equal(st_l.slot_token, st_s.slot_token)
    assert np.array_equal(st_l.slot_stamp, st_s.slot_stamp)
    assert np.array_equal(st_l.tok2slot, st_s.tok2slot)


def test_pool_exhaustion_and_missing_block_are_errors():
    bt, hbt = _tables(4, set(), 0)
    st = oracle.HotState.cold(128, 4 * BLOCK)
    hot = np.full(2, -1, np.int32)
    pool = oracle.HotPool([5])
    oracle.resolve(np.arange(64, dtype=np.int32)[None], bt, hbt, hot, st, pool)   # one page
    assert list(hot) == [5, -1] and pool.free == []
    with pytest.raises(ResolveError):
        oracle.resolve(np.arange(64, 65 + 64, dtype=np.int32)[None], bt, hbt, hot, st, pool)
    st2 = oracle.HotState.cold(128, 4 * BLOCK)
    with pytest.raises(ResolveError):                               # no pool, no block
        oracle.resolve(np.array([[3]], np.int32), bt, hbt, np.full(2, -1, np.int32), st2)


def test_release_makes_the_request_cold():
    bt, hbt = _tables(6, set(), 0)
    pool = oracle.HotPool([7, 8, 9])
    st = oracle.HotState.cold(128, 6 * BLOCK)
    hot = np.full(2, -1, np.int32)
    oracle.resolve(np.arange(0, 100, dtype=np.int32)[None], bt, hbt, hot, st, pool)
    assert list(hot) == [7, 8] and pool.free == [9]
    back = oracle.release_hot(st, hot, pool)
    assert back == [7, 8] and pool.free == [9, 7, 8] and list(hot) == [-1, -1]
    assert (st.slot_token == -1).all() and (st.slot_stamp == -1).all() and (st.tok2slot == -1).all()
    # the same tokens again: every one a miss, filled from slot 0, on blocks from the front
    rows, copies, stats = oracle.resolve(np.arange(0, 100, dtype=np.int32)[None], bt, hbt, hot, st, pool)
    assert stats[1:3] == (0, 100) and [c[1] for c in copies] == list(range(100))
    assert list(hot) == [9, 7] and rows[0, 0] == 9 * BLOCK and rows[0, 99] == 7 * BLOCK + 35
    # without a pool only the state is cleared and the blocks stay
    hot2 = np.array([3, 4], np.int32)
    st2 = oracle.HotState.cold(128, 6 * BLOCK)
    oracle.resolve(np.arange(0, 10, dtype=np.int32)[None], bt, hbt, hot2, st2)
    assert oracle.release_hot(st2, hot2) == [] and list(hot2) == [3, 4]
    assert (st2.tok2slot == -1).all() and st2.step == 0


@pytest.mark.parametrize("seed", [3, 4])
def test_plan_windows_equal_pinned_lru_model(seed):
    # calls inside one window never take a slot touched earlier in the window; every plan of the
    # window still reads its own tokens when the window ends (the plans can be replayed)
    rng = np.random.default_rng(seed)
    H, n_pages = 320, 14
    resident_pages = {13}
    resident = {t for t in range(13 * BLOCK, 14 * BLOCK)}
    bt, hbt = _tables(n_pages, resident_pages, 0)
    hot = np.arange(20, 20 + H // BLOCK, dtype=np.int32)
    model = LeaseModel(H, [])
    model._r(0)["pages"] = [int(x) for x in hot]
    st = oracle.HotState.cold(H, n_pages * BLOCK)
    window_start, plans = None, []
    replayed = 0
    for call in range(80):
        begin = call % 4 == 0 or rng.random() < 0.15               # windows of 1 to 4 calls
        if begin:
            for topk, rows in plans:                                # end of the previous window
                for j in range(topk.shape[0]):
                    for k in range(topk.shape[1]):
                        t = int(topk[j, k])
                        if t >= 0 and t not in resident:
                            s = ((int(rows[j, k]) // BLOCK - 20) * BLOCK) + int(rows[j, k]) % BLOCK
                            assert st.slot_token[s] == t
                            replayed += 1
            plans = []
            window_start = st.step
        n = int(rng.integers(1, 75))
        U = rng.choice(n_pages * BLOCK, n, replace=False)
        topk = _topk(U, 1 + call % 3, rng)
        expect = model.call(0, U, resident, begin=begin)
        rows, _, _ = oracle.resolve(topk, bt, hbt, hot, st, window_start=window_start)
        assert list(st.slot_token) == model.req[0]["slot_token"]
        for j in range(topk.shape[0]):
            for k in range(topk.shape[1]):
                t = int(topk[j, k])
                if t >= 0 and t not in resident:
                    assert rows[j, k] == expect[t]
        plans.append((topk, rows))
    assert replayed > 0


def test_window_larger_than_the_hot_buffer_is_an_error():
    bt, hbt = _tables(8, set(), 0)
    hot = np.arange(2, dtype=np.int32)
    st = oracle.HotState.cold(128, 8 * BLOCK)
    oracle.resolve(np.arange(0, 100, dtype=np.int32)[None], bt, hbt, hot, st, window_start=0)
    # a second call of the same window may not evict the first call's 100 rows
    with pytest.raises(ResolveError):
        oracle.resolve(np.arange(100, 130, dtype=np.int32)[None], bt, hbt, hot, st, window_start=0)
    st2 = oracle.HotState.cold(128, 8 * BLOCK)
    oracle.resolve(np.arange(0, 100, dtype=np.int32)[None], bt, hbt, hot, st2, window_start=0)
    oracle.resolve(np.arange(100, 130, dtype=np.int32)[None], bt, hbt, hot, st2)  # a new window: fine
