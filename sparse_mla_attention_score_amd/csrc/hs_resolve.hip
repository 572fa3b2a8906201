// Fused top-K resolver and hot-buffer state (gfx950).
//
// What is computed (Hybrid HiSparse part-1 page, "How it works", hybrid residency bullet and
// the paragraph that follows it): each token selected by the indexer is read where it lives.
// A token on a GPU-resident page is read in place.  A token in the token-indexed hot buffer
// is read there and its LRU entry is refreshed.  Any other token is a miss: its single row
// is copied from pinned host memory into an LRU slot of the hot buffer.  The hot buffer's
// pages are ordinary blocks of the shared KV pool, so every selected row is named by one row
// id into one tensor with one stride.  Nothing waits on the CPU.
//
// Readings where the pages are silent (the same ones the oracle takes): the LRU clock is the
// request's resolve-call counter; a hit and a fill both stamp it; resident pages win and do
// not touch the LRU; victims are the slots untouched in this call in (stamp, slot) order,
// empty slots first; the i-th miss in ascending token order takes the i-th victim.
//
// Implementation: one 1,024-thread workgroup per request decides, a second kernel copies.  The
// S top-K lists become their sorted union through a token bitmap of the request.  The (stamp, slot) order is kept as
// an explicit recency list of slots, double-buffered by the parity of the call counter: the
// victims are the first untouched entries of the old list, and the new list is the untouched
// entries in old order followed by the touched slots in ascending slot order, which is the
// (stamp, slot) order after this call.  Every choice is a prefix sum, so the result does not
// depend on thread timing.  Each request's miss list then goes to a copy kernel that spreads
// the rows of the whole batch over the GPU (one request's misses alone cannot fill the host
// link), reading the mapped host pool directly, all layers sharing the request's top-K.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kResThreads = 1024;
constexpr int kPerU = kMaxUnion / kResThreads;  // union entries per thread, at most
constexpr int kPerH = kMaxHot / kResThreads;    // hot slots per thread, at most

// Number of entries of the ascending list a[0..n) that are < x, or <= x when or_equal.
__device__ __forceinline__ int count_below(const int32_t* a, int n, int32_t x, bool or_equal) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int32_t v = a[mid];
    if (v < x || (or_equal && v == x)) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Sum of v over the block, added to *dst (one LDS atomic per wave).
__device__ __forceinline__ void block_add(int v, int* dst) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(dst, v);
}

__global__ __launch_bounds__(kResThreads) void resolve_kernel(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ ctx_lens, int S, int K,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ host_block_table,
    const int32_t* __restrict__ hot_blocks, int max_pages, int H, int64_t num_gpu_blocks,
    int64_t num_host_blocks, int max_batch, int32_t* __restrict__ slot_token,
    int32_t* __restrict__ slot_stamp, int32_t* __restrict__ lru_order,
    int32_t* __restrict__ tok2slot, int64_t lmax, int32_t* __restrict__ req_step,
    int32_t* __restrict__ req_used, int32_t* __restrict__ miss_src, int32_t* __restrict__ miss_dst,
    int32_t* __restrict__ miss_cnt, int union_cap, int32_t* __restrict__ row_ids,
    int32_t* __restrict__ stats, uint32_t* __restrict__ ubits, int64_t ubits_stride,
    int tables_off, const int32_t* __restrict__ begin_window, int32_t* __restrict__ win_start,
    int leasing, int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char dyn[];
  // union_cap (a power of two, >= S*K and >= 1024) entries each: sorted union U, per-entry
  // class `cls` (row id, -1, or -2 - miss rank), the token of each miss (then its host row),
  // each miss's victim slot (then its row); then H slot flags; then, when they fit
  // (tables_off > 0), copies of the request's block table and host block table.
  int32_t* U = reinterpret_cast<int32_t*>(dyn);
  int32_t* cls = U + union_cap;
  int32_t* msrc = cls + union_cap;
  int32_t* mdst = msrc + union_cap;
  uint8_t* flag = reinterpret_cast<uint8_t*>(mdst + union_cap);
  __shared__ int32_t lhot[kMaxHot / kBlock];
  __shared__ int scan[kResThreads / 64 + 1];
  __shared__ int cnt[8];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int Lb = ctx_lens[b];
  const int step = req_step[b];
  // Plan window: slots touched by a call of the current window (stamp >= protect) are never
  // given to a miss.  A call that begins a window protects only its own hits.
  const bool begin = begin_window == nullptr || begin_window[b] != 0;
  const int protect = begin ? step : min(win_start[b], step);
  const bool windowed = protect < step;
  const int32_t* tk = topk + (int64_t)b * S * K;
  int32_t* out = row_ids + (int64_t)b * S * K;
  const int32_t* bt = block_table + (int64_t)b * max_pages;
  const int32_t* hbt = host_block_table + (int64_t)b * max_pages;
  const int32_t* hot = hot_blocks + (int64_t)b * (H / kBlock);
  int32_t* st_tok = slot_token + (int64_t)b * H;
  int32_t* st_stamp = slot_stamp + (int64_t)b * H;
  int32_t* t2s = tok2slot + (int64_t)b * lmax;
  const int32_t* order_cur = lru_order + ((int64_t)(step & 1) * max_batch + b) * H;
  int32_t* order_next = lru_order + ((int64_t)((step + 1) & 1) * max_batch + b) * H;

  if (Lb < S || Lb > max_pages * kBlock) {
    if (tid == 0) {
      raise_error(err, HS_DEVERR_SHORT_CONTEXT);
      miss_cnt[b] = 0;
    }
    for (int i = tid; i < S * K; i += kResThreads) out[i] = -1;
    return;
  }

  // Everything that depends only on the inputs is loaded up front and kept in registers: the
  // thread's entries of the S lists (i = tid + 1024 e; used again for the row ids) and its
  // run of the recency list.
  const int n_in = S * K;
  const int perH = (H + kResThreads - 1) / kResThreads;  // <= kPerH
  const int h0 = tid * perH;
  int32_t tkv[kPerU], ord[kPerH], ost[kPerH];
#pragma unroll
  for (int e = 0; e < kPerU; ++e) tkv[e] = tid + e * kResThreads < n_in ? tk[tid + e * kResThreads] : -1;
#pragma unroll
  for (int e = 0; e < kPerH; ++e) ord[e] = e < perH && h0 + e < H ? order_cur[h0 + e] : -1;
  // inside a window, the stamps of the listed slots (before this call) decide which are free
#pragma unroll
  for (int e = 0; e < kPerH; ++e) ost[e] = windowed && ord[e] >= 0 && ord[e] < H ? st_stamp[ord[e]] : -1;
  for (int i = tid; i < H / kBlock; i += kResThreads) lhot[i] = hot[i];
  // The page tables are read per union entry (up to 8 per thread, at random pages): from LDS
  // when they fit, staged here with coalesced loads.
  const int n_pages = (Lb + kBlock - 1) / kBlock;
  int32_t* lbt = tables_off > 0 ? reinterpret_cast<int32_t*>(dyn + tables_off) : nullptr;
  int32_t* lhbt = lbt ? lbt + max_pages : nullptr;
  if (lbt) {
    for (int i = tid; i < n_pages; i += kResThreads) {
      lbt[i] = bt[i];
      lhbt[i] = hbt[i];
    }
  }
  const int32_t* pbt = lbt ? lbt : bt;
  const int32_t* phbt = lbt ? lhbt : hbt;

  // ---- 1. sorted union of the S lists through a token bitmap of the request: a bit per
  // selected token, then the set bits read out in order.  The bitmap lives in LDS (over msrc
  // and mdst, free until step 2) when the context fits, else in workspace scratch.  Padding
  // (-1) is skipped; tokens outside [0, Lb) are flagged and skipped.
  const int n_words = (Lb + 31) >> 5;
  if (tid < 8) cnt[tid] = 0;
  for (int i = tid; i < H; i += kResThreads) flag[i] = 0;
  int nU;
  // wpre (when given): each word's first place in U, so that a token's place is its word's
  // plus the set bits below it in the word
  auto read_out = [&](auto word_at, int32_t* wpre) {
    const int per = (n_words + kResThreads - 1) / kResThreads;
    const int w0 = min(n_words, tid * per), w1 = min(n_words, w0 + per);
    int c = 0;
    for (int wd = w0; wd < w1; ++wd) c += __popc(word_at(wd));
    int tot;
    int pos = block_exclusive_scan<kResThreads>(c, scan, &tot);
    for (int wd = w0; wd < w1; ++wd) {
      uint32_t v = word_at(wd);
      if (wpre) wpre[wd] = pos;
      while (v) {
        const int bit = __ffs(v) - 1;
        v &= v - 1;
        U[pos++] = wd * 32 + bit;
      }
    }
    nU = tot;
  };
  auto mark = [&](uint32_t* words) {
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      const int32_t t = tkv[e];
      if (t >= Lb) raise_error(err, HS_DEVERR_BAD_ROW);
      else if (t >= 0) atomicOr(&words[t >> 5], 1u << (t & 31));
    }
  };
  // One list (S = 1): if its valid tokens are strictly ascending and its padding comes only at
  // the end (as the top-K call emits it), the list is already the sorted union, and the bitmap
  // is skipped.  Any other list takes the bitmap below.
  bool direct = false;
  // upos: the place in U of each of the thread's list entries, when it is known before step 5
  // (else step 5 finds it by binary search)
  int32_t upos[kPerU];
  bool have_pos = false;
  if (S == 1) {
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      const int i = tid + e * kResThreads;
      if (i < n_in) U[i] = tkv[e];
    }
    __syncthreads();
    int bad = 0, valid = 0;
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      const int i = tid + e * kResThreads;
      if (i >= n_in) continue;
      const int32_t t = tkv[e], prev = i > 0 ? U[i - 1] : -1;
      if (t >= 0) {
        valid += 1;
        if (t >= Lb || (i > 0 && prev >= t) || (i > 0 && prev < 0)) bad = 1;  // out of range, unordered, or after padding
      }
    }
    __shared__ int n_valid;
    if (tid == 0) n_valid = 0;
    bad = __syncthreads_or(bad);
    block_add(valid, &n_valid);
    __syncthreads();
    if (!bad) {
      direct = true;
      nU = n_valid;
    }
  }
  if (direct) {
    // U holds the list: entry i is at place i
#pragma unroll
    for (int e = 0; e < kPerU; ++e) upos[e] = tid + e * kResThreads;
    have_pos = true;
  } else if (n_words <= 2 * union_cap) {
    uint32_t* lb = reinterpret_cast<uint32_t*>(msrc);
    for (int i = tid; i < n_words; i += kResThreads) lb[i] = 0u;
    __syncthreads();
    mark(lb);
    __syncthreads();
    // with the bitmap in msrc alone, the words' first places fit in cls (free until step 2)
    int32_t* wpre = n_words <= union_cap ? cls : nullptr;
    read_out([&](int wd) { return lb[wd]; }, wpre);
    if (wpre) {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kPerU; ++e) {
        const int32_t t = tkv[e];
        upos[e] = t >= 0 && t < Lb ? wpre[t >> 5] + __popc(lb[t >> 5] & ((1u << (t & 31)) - 1u)) : 0;
      }
      have_pos = true;
    }
  } else {
    uint32_t* ub = ubits + (int64_t)b * ubits_stride;
    for (int i = tid; i < n_words; i += kResThreads) ub[i] = 0u;
    __syncthreads();  // the zeroing stores have completed before any bit is set
    mark(ub);
    __syncthreads();  // the atomics were performed in L2; the words are read back at agent scope
    read_out([&](int wd) { return load_agent(&ub[wd]); }, nullptr);
  }
  __syncthreads();

  // ---- 2. classify: resident / hot hit (stamped) / miss.  Thread owns a contiguous run.
  int n_miss;
  {
    const int per = (nU + kResThreads - 1) / kResThreads;  // <= kPerU
    const int i0 = tid * per;
    int32_t u[kPerU], blk[kPerU], slot[kPerU], hb[kPerU];
    int n_res = 0, n_hit = 0, my_miss = 0;
    // the three lookups of a token are independent loads, issued together (one round trip);
    // only the one its class needs is used
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      u[e] = -1;
      blk[e] = slot[e] = hb[e] = -1;
      if (e < per && i0 + e < nU) {
        u[e] = U[i0 + e];
        blk[e] = pbt[u[e] >> 6];
        slot[e] = t2s[u[e]];
        hb[e] = phbt[u[e] >> 6];
      }
    }
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      if (u[e] < 0) continue;
      int32_t c = -1;
      if (blk[e] >= 0) {
        if (blk[e] < num_gpu_blocks) c = blk[e] * kBlock + (u[e] & 63);
        else raise_error(err, HS_DEVERR_BAD_BLOCK);
        ++n_res;
      } else if (slot[e] >= 0 && slot[e] < H) {
        const int32_t s = slot[e];
        flag[s] = 1;  // stamped with the other touched slots in step 3
        const int32_t h = lhot[s >> 6];
        if (h >= 0 && h < num_gpu_blocks) c = h * kBlock + (s & 63);
        else raise_error(err, HS_DEVERR_BAD_BLOCK);
        ++n_hit;
      } else if (hb[e] < 0) {
        raise_error(err, HS_DEVERR_NO_HOST_COPY);
      } else if (hb[e] >= num_host_blocks) {
        raise_error(err, HS_DEVERR_BAD_BLOCK);
      } else {
        c = -2;  // miss; rank assigned below
        ++my_miss;
      }
      cls[i0 + e] = c;
    }
    block_add(n_res, &cnt[0]);
    block_add(n_hit, &cnt[1]);
    int tot;
    int rank = block_exclusive_scan<kResThreads>(my_miss, scan, &tot);
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      if (u[e] >= 0 && cls[i0 + e] == -2) {
        cls[i0 + e] = -2 - rank;  // miss code carries its rank (ascending token order)
        msrc[rank] = u[e];
        ++rank;
      }
    }
    n_miss = tot;
  }

  // ---- 3. victims: the first n_miss slots of the recency list untouched in this call (and,
  // inside a window, in the window's earlier calls), then the new list (untouched slots in old
  // order, then every slot touched by this call in ascending slot order)
  int n_assign;
  {
    auto free_slot = [&](int e) {
      return ord[e] >= 0 && ord[e] < H && !flag[ord[e]] && (!windowed || ost[e] < protect);
    };
    int my_cand = 0;
#pragma unroll
    for (int e = 0; e < kPerH; ++e)
      if (free_slot(e)) ++my_cand;
    int tot;
    int r = block_exclusive_scan<kResThreads>(my_cand, scan, &tot);
#pragma unroll
    for (int e = 0; e < kPerH; ++e) {
      if (free_slot(e)) {
        if (r < n_miss) mdst[r] = ord[e];
        ++r;
      }
    }
    n_assign = min(n_miss, tot);
    if (tid == 0 && n_assign < n_miss) raise_error(err, HS_DEVERR_HOT_FULL);
  }
  __syncthreads();
  for (int r = tid; r < n_assign; r += kResThreads) flag[mdst[r]] = 1;
  __syncthreads();
  {
    // both counts in one scan: kept slots in the low 16 bits, touched in the high 16 (each
    // total is at most H <= 16,384, so the halves never carry into each other).  Every touched
    // slot (hit or victim) takes this call's stamp here, in the thread's contiguous run.
    int packed = 0;
#pragma unroll
    for (int e = 0; e < kPerH; ++e) {
      if (ord[e] >= 0 && ord[e] < H && !flag[ord[e]]) packed += 1;
      if (e < perH && h0 + e < H && flag[h0 + e]) {
        packed += 1 << 16;
        st_stamp[h0 + e] = step;
      }
    }
    int tot;
    const int pre = block_exclusive_scan<kResThreads>(packed, scan, &tot);
    const int n_keep = tot & 0xffff;
    int pk = pre & 0xffff, pt = n_keep + (pre >> 16);
#pragma unroll
    for (int e = 0; e < kPerH; ++e) {
      if (ord[e] >= 0 && ord[e] < H && !flag[ord[e]]) order_next[pk++] = ord[e];
      if (e < perH && h0 + e < H && flag[h0 + e]) order_next[pt++] = h0 + e;
    }
  }

  // ---- 4. fill the victims (rank order = ascending token order) and publish the miss list;
  // the copy kernel moves the rows
  int fills = 0;
  for (int r = tid; r < n_assign; r += kResThreads) {
    const int32_t u = msrc[r];
    const int32_t v = mdst[r];
    const int32_t old = st_tok[v];
    const int32_t hbk = phbt[u >> 6];  // checked in step 2
    if (old >= 0 && old < lmax) t2s[old] = -1;
    else ++fills;
    st_tok[v] = u;
    t2s[u] = v;
    const int32_t h = lhot[v >> 6];
    int32_t row = -1;
    if (h >= 0 && h < num_gpu_blocks) row = h * kBlock + (v & 63);
    else if (leasing && h < 0) row = -2 - v;  // the page leases its block after this kernel
    else raise_error(err, HS_DEVERR_BAD_BLOCK);
    mdst[r] = row;
    miss_src[(int64_t)b * n_in + r] = hbk * kBlock + (u & 63);
    miss_dst[(int64_t)b * n_in + r] = row;
  }
  block_add(fills, &cnt[2]);
  if (tid == 0) miss_cnt[b] = n_assign;
  __syncthreads();

  // ---- 5. row ids, positionally: each entry's place in U, known from step 1 or found by
  // binary search (the thread's searches advance together, one LDS round trip per halving step)
  {
    int lo[kPerU], hi[kPerU];
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      lo[e] = have_pos ? upos[e] : 0;
      hi[e] = have_pos ? upos[e] : tkv[e] >= 0 && tkv[e] < Lb ? nU : 0;
    }
    for (int it = 0; !have_pos && (1 << it) <= nU; ++it) {
#pragma unroll
      for (int e = 0; e < kPerU; ++e) {
        if (lo[e] < hi[e]) {
          const int mid = (lo[e] + hi[e]) >> 1;
          if (U[mid] < tkv[e]) lo[e] = mid + 1;
          else hi[e] = mid;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kPerU; ++e) {
      const int i = tid + e * kResThreads;
      if (i >= n_in) continue;
      int32_t r = -1;
      if (tkv[e] >= 0 && tkv[e] < Lb && nU > 0) {
        const int32_t c = cls[lo[e]];
        if (c >= -1) r = c;
        else if (-2 - c < n_assign) r = mdst[-2 - c];
      }
      out[i] = r;
    }
  }
  if (tid == 0) {
    const int used = min(H, req_used[b] + cnt[2]);
    req_used[b] = used;
    req_step[b] = step + 1;
    if (begin) win_start[b] = step;
    if (stats) {
      stats[b * 4 + 0] = cnt[0];
      stats[b * 4 + 1] = cnt[1];
      stats[b * 4 + 2] = n_miss;
      stats[b * 4 + 3] = (used + kBlock - 1) / kBlock;
    }
  }
}

// Leases of one resolve call (hot_leasing): every hot page below a request's filled slots that
// has no block yet takes the next block of the free-block pool, request by request, page by
// page (a scan over the flattened (request, page) order keeps that order with any number of
// threads).  An empty pool leaves the page at -1 and flags the call.
constexpr int kLeaseThreads = 1024;

__global__ __launch_bounds__(kLeaseThreads) void lease_kernel(
    int B, int pages_per_req, const int32_t* __restrict__ req_used, int32_t* __restrict__ hot_blocks,
    const int32_t* __restrict__ ring, int64_t* __restrict__ ctr, int64_t cap, int64_t num_gpu_blocks,
    int32_t* __restrict__ err) {
  __shared__ int scan[kLeaseThreads / 64 + 1];
  const int64_t head = ctr[0], avail = ctr[1] - ctr[0];
  const int total = B * pages_per_req;
  int64_t carry = 0;
  for (int base = 0; base < total; base += kLeaseThreads) {
    const int f = base + (int)threadIdx.x;
    int need = 0;
    if (f < total) {
      const int b = f / pages_per_req, p = f - b * pages_per_req;
      const int used = min(max(req_used[b], 0), pages_per_req * kBlock);
      need = p < (used + kBlock - 1) / kBlock && hot_blocks[f] < 0;
    }
    int tot;
    const int x = block_exclusive_scan<kLeaseThreads>(need, scan, &tot);
    if (need) {
      const int64_t pos = carry + x;
      if (pos < avail) {
        const int32_t blk = ring[(head + pos) % cap];
        if (blk >= 0 && blk < num_gpu_blocks) hot_blocks[f] = blk;
        else raise_error(err, HS_DEVERR_BAD_BLOCK);
      } else {
        raise_error(err, HS_DEVERR_POOL_EMPTY);
      }
    }
    carry += tot;
  }
  if (threadIdx.x == 0) ctr[0] = head + (carry < avail ? carry : avail);
}

// Single-row copies of every miss of the batch, spread over the whole grid: host row
// miss_src -> device row miss_dst, for every layer, 16 bytes per work item, eight loads in
// flight per thread.  Rows whose destination is invalid (-1) are skipped.  With leasing, a
// destination on a page leased after the resolver ran is given as -2 - slot and is looked up
// in the hot-page table here, and the row ids the resolver left in that form are rewritten.
constexpr int kCopyThreads = 256;
constexpr int kCopyBlocks = 256;

__global__ __launch_bounds__(kCopyThreads) void miss_copy_kernel(
    const int32_t* __restrict__ miss_src, const int32_t* __restrict__ miss_dst,
    const int32_t* __restrict__ miss_cnt, int B, int per_req, const uint8_t* __restrict__ host_pool,
    uint8_t* __restrict__ kv_pool, int n_layers, int row_bytes, int64_t num_gpu_blocks,
    int64_t num_host_blocks, const int32_t* __restrict__ hot_blocks, int pages_per_req,
    int32_t* __restrict__ row_ids, int64_t n_row_ids, int row_ids_per_req) {
  __shared__ int scan[kCopyThreads / 64 + 1];
  // prefix sums of the per-request miss counts (B may exceed the block: chunks with carry)
  extern __shared__ int req_start[];  // [B + 1]
  int carry = 0;
  for (int base = 0; base < B; base += kCopyThreads) {
    const int i = base + threadIdx.x;
    const int v = i < B ? min(max(miss_cnt[i], 0), per_req) : 0;
    int tot;
    const int x = block_exclusive_scan<kCopyThreads>(v, scan, &tot);
    if (i < B) req_start[i] = carry + x;
    carry += tot;
  }
  if (threadIdx.x == 0) req_start[B] = carry;
  __syncthreads();
  const int chunks = row_bytes / 16;
  const int per_row = n_layers * chunks;
  const int64_t total = (int64_t)carry * per_row;
  const int64_t gpu_layer = num_gpu_blocks * kBlock * (int64_t)row_bytes;
  const int64_t host_layer = num_host_blocks * kBlock * (int64_t)row_bytes;
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads;
  constexpr int kBatch = 8;
  for (int64_t base = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; base < total;
       base += stride * kBatch) {
    u32x4 v[kBatch];
    int64_t dst[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int64_t idx = base + e * stride;
      dst[e] = -1;
      if (idx < total) {
        const int row = (int)(idx / per_row);
        const int rem = (int)(idx - (int64_t)row * per_row);
        const int layer = rem / chunks, q = rem - layer * chunks;
        int lo = 0, hi = B - 1;  // request whose range holds `row`
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (req_start[mid] <= row) lo = mid;
          else hi = mid - 1;
        }
        const int64_t k = (int64_t)lo * per_req + (row - req_start[lo]);
        const int32_t s = miss_src[k];
        int32_t d = miss_dst[k];
        if (hot_blocks && d <= -2) {
          const int v = -2 - d;
          const int32_t blk = hot_blocks[(int64_t)lo * pages_per_req + (v >> 6)];
          d = blk >= 0 ? blk * kBlock + (v & 63) : -1;
        }
        if (d >= 0 && d < num_gpu_blocks * kBlock && s >= 0 && s < num_host_blocks * kBlock) {
          v[e] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(host_pool + layer * host_layer + (int64_t)s * row_bytes + q * 16));
          dst[e] = layer * gpu_layer + (int64_t)d * row_bytes + q * 16;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e)
      if (dst[e] >= 0) *reinterpret_cast<u32x4*>(kv_pool + dst[e]) = v[e];
  }
  if (hot_blocks) {
    for (int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n_row_ids; i += stride) {
      const int32_t r = row_ids[i];
      if (r > -2) continue;
      const int v = -2 - r;
      const int32_t blk = hot_blocks[(i / row_ids_per_req) * pages_per_req + (v >> 6)];
      row_ids[i] = blk >= 0 ? blk * kBlock + (v & 63) : -1;
    }
  }
}

// Requests' hot buffers made cold (hs_hot_release): one workgroup per listed request clears its
// slots, recency lists, token-to-slot entries (through the tokens its slots hold), counters and
// top-K guesses.  A request listed twice is cleared twice, to the same state.
__global__ __launch_bounds__(256) void hot_release_kernel(
    const int32_t* __restrict__ reqs, int max_batch, int H, int max_queries,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_stamp,
    int32_t* __restrict__ lru_order, int32_t* __restrict__ tok2slot, int64_t lmax,
    int32_t* __restrict__ req_step, int32_t* __restrict__ req_used, int32_t* __restrict__ win_start,
    uint32_t* __restrict__ guess, int32_t* __restrict__ err) {
  const int b = reqs[blockIdx.x];
  if (b < 0 || b >= max_batch) {
    if (threadIdx.x == 0) raise_error(err, HS_DEVERR_BAD_REQUEST);
    return;
  }
  int32_t* st_tok = slot_token + (int64_t)b * H;
  int32_t* t2s = tok2slot + (int64_t)b * lmax;
  for (int s = threadIdx.x; s < H; s += blockDim.x) {
    const int32_t u = st_tok[s];
    if (u >= 0 && u < lmax) t2s[u] = -1;
    st_tok[s] = -1;
    slot_stamp[(int64_t)b * H + s] = -1;
    lru_order[(int64_t)b * H + s] = s;
    lru_order[((int64_t)max_batch + b) * H + s] = s;
  }
  if (threadIdx.x == 0) {
    req_step[b] = 0;
    req_used[b] = 0;
    win_start[b] = 0;
  }
  if (threadIdx.x < max_queries) guess[b * max_queries + threadIdx.x] = kGuessOff;
}

// The free-block pool's sequential updates, one wave: blocks of released requests (page order,
// list order) or given blocks appended at the back.  A released request's pages are cleared
// as they are returned, so a request listed twice returns its blocks once.
__global__ __launch_bounds__(64) void pool_append_kernel(
    const int32_t* __restrict__ list, int n, int from_requests, int max_batch, int pages_per_req,
    int32_t* __restrict__ hot_blocks, int32_t* __restrict__ ring, int64_t* __restrict__ ctr,
    int64_t cap, int64_t num_gpu_blocks, int32_t* __restrict__ err) {
  const int lane = threadIdx.x;
  const int64_t head = ctr[0];
  int64_t tail = ctr[1];
  auto push = [&](int32_t blk, bool ok) {
    const uint64_t m = __ballot(ok);
    const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    const int64_t room = cap - (tail - head);
    if (ok) {
      if (pos < room) ring[(tail + pos) % cap] = blk;
      else raise_error(err, HS_DEVERR_POOL_FULL);
    }
    const int64_t cnt = __popcll(m);
    tail += cnt < room ? cnt : room;
  };
  if (from_requests) {
    for (int i = 0; i < n; ++i) {
      const int b = list[i];
      if (b < 0 || b >= max_batch) continue;  // flagged by hot_release_kernel
      for (int p0 = 0; p0 < pages_per_req; p0 += 64) {
        const int p = p0 + lane;
        int32_t* e = hot_blocks + (int64_t)b * pages_per_req + p;
        const int32_t blk = p < pages_per_req ? *e : -1;
        push(blk, blk >= 0);
        if (blk >= 0) *e = -1;
      }
    }
  } else {
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int32_t blk = i0 + lane < n ? list[i0 + lane] : -1;
      if (blk >= num_gpu_blocks) raise_error(err, HS_DEVERR_BAD_BLOCK);
      push(blk, blk >= 0 && blk < num_gpu_blocks);
    }
  }
  if (lane == 0) ctr[1] = tail;
}

__global__ void hot_reset_kernel(int32_t* slot_token, int32_t* slot_stamp, int32_t* lru_order,
                                 int64_t n_slots, int H, int32_t* tok2slot, int64_t n_tok,
                                 int32_t* req_step, int32_t* req_used, int32_t* win_start,
                                 int max_batch, uint32_t* guess,
                                 int n_guess, unsigned long long* path_count, int32_t* hot_blocks,
                                 int64_t n_hot_blocks, int64_t* pool_ctr, int64_t n_all,
                                 int32_t* err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_all; i += stride) {
    if (i < n_tok) tok2slot[i] = -1;
    if (i < n_slots) {
      slot_token[i] = -1;
      slot_stamp[i] = -1;
      lru_order[i] = (int32_t)(i % H);
      lru_order[n_slots + i] = (int32_t)(i % H);
    }
    if (i < n_guess) guess[i] = kGuessOff;
    if (i < 2) path_count[i] = 0;
    if (i < max_batch) {
      req_step[i] = 0;
      req_used[i] = 0;
      win_start[i] = 0;
    }
    if (i < n_hot_blocks) hot_blocks[i] = -1;  // only with leasing (n_hot_blocks = 0 otherwise)
    if (pool_ctr && i < 2) pool_ctr[i] = 0;
    if (i == 0) *err = 0;
  }
}

}  // namespace
}  // namespace hs

using namespace hs;

static int union_cap_for(int S, int K) {
  int n = 1;
  while (n < S * K) n <<= 1;
  return n < 1024 ? 1024 : n;
}

// Dynamic LDS of the resolver: the union arrays and the slot flags, plus both page tables of
// a request when everything fits a CU's 160 KiB (less a margin for the static arrays).
static size_t resolve_lds_base(int S, int K, int H) {
  return (size_t)union_cap_for(S, K) * 16 + (size_t)((H + 15) / 16) * 16;
}

static size_t resolve_lds_with_tables(int S, int K, int H, int max_pages) {
  const size_t base = resolve_lds_base(S, K, H);
  const size_t with = base + (size_t)max_pages * 8;
  return with <= 160 * 1024 - 2048 ? with : base;
}

hipError_t hs_launch_resolve(const hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens, int B,
                             int S, const int32_t* begin_window, int32_t* row_ids, int32_t* stats,
                             hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  const int H = ctx->lay.hot_rows;
  const int cap = union_cap_for(S, c.topk);
  const size_t base = resolve_lds_base(S, c.topk, H);
  const size_t lds = resolve_lds_with_tables(S, c.topk, H, c.max_pages_per_req);
  const int tables_off = lds > base ? (int)base : 0;
  hs_timer_mark(ctx, HS_KERNEL_RESOLVE, true, stream);
  hipLaunchKernelGGL(resolve_kernel, dim3((unsigned)B), dim3(kResThreads), lds, stream, topk,
                     ctx_lens, S, c.topk, ctx->buf.block_table, ctx->buf.host_block_table,
                     ctx->buf.hot_blocks, c.max_pages_per_req, H, (int64_t)c.num_gpu_blocks,
                     (int64_t)c.num_host_blocks, c.max_batch, ctx->ws.slot_token,
                     ctx->ws.slot_stamp, ctx->ws.lru_order, ctx->ws.tok2slot, ctx->lay.lmax,
                     ctx->ws.req_step, ctx->ws.req_used, ctx->ws.miss_src, ctx->ws.miss_dst,
                     ctx->ws.miss_cnt, cap, row_ids, stats, ctx->ws.bitmap,
                     (int64_t)c.max_queries * ctx->lay.bm_words, tables_off, begin_window,
                     ctx->ws.win_start, c.hot_leasing, ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_RESOLVE, false, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.num_host_blocks == 0) return e;
  const int pages_per_req = H / kBlock;
  if (c.hot_leasing) {
    hs_timer_mark(ctx, HS_KERNEL_LEASE, true, stream);
    hipLaunchKernelGGL(lease_kernel, dim3(1), dim3(kLeaseThreads), 0, stream, B, pages_per_req,
                       ctx->ws.req_used, ctx->buf.hot_blocks, ctx->ws.pool_ring, ctx->ws.pool_ctr,
                       (int64_t)c.num_gpu_blocks, (int64_t)c.num_gpu_blocks, ctx->ws.err);
    hs_timer_mark(ctx, HS_KERNEL_LEASE, false, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hs_timer_mark(ctx, HS_KERNEL_MISS_COPY, true, stream);
  hipLaunchKernelGGL(miss_copy_kernel, dim3(kCopyBlocks), dim3(kCopyThreads), (size_t)(B + 1) * 4,
                     stream, ctx->ws.miss_src, ctx->ws.miss_dst, ctx->ws.miss_cnt, B, S * c.topk,
                     static_cast<const uint8_t*>(ctx->host_pool_dev),
                     static_cast<uint8_t*>(ctx->buf.kv_pool), c.n_layers, ctx->row_bytes,
                     (int64_t)c.num_gpu_blocks, (int64_t)c.num_host_blocks,
                     c.hot_leasing ? ctx->buf.hot_blocks : nullptr, pages_per_req, row_ids,
                     (int64_t)B * S * c.topk, S * c.topk);
  hs_timer_mark(ctx, HS_KERNEL_MISS_COPY, false, stream);
  return hipGetLastError();
}

hipError_t hs_launch_hot_release(const hs_ctx* ctx, const int32_t* reqs, int n, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  const int H = ctx->lay.hot_rows;
  if (c.hot_leasing) {
    hs_timer_mark(ctx, HS_KERNEL_POOL_GIVE, true, stream);
    hipLaunchKernelGGL(pool_append_kernel, dim3(1), dim3(64), 0, stream, reqs, n, 1, c.max_batch,
                       H / kBlock, ctx->buf.hot_blocks, ctx->ws.pool_ring, ctx->ws.pool_ctr,
                       (int64_t)c.num_gpu_blocks, (int64_t)c.num_gpu_blocks, ctx->ws.err);
    hs_timer_mark(ctx, HS_KERNEL_POOL_GIVE, false, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hs_timer_mark(ctx, HS_KERNEL_HOT_RELEASE, true, stream);
  hipLaunchKernelGGL(hot_release_kernel, dim3((unsigned)n), dim3(256), 0, stream, reqs, c.max_batch,
                     H, c.max_queries, ctx->ws.slot_token, ctx->ws.slot_stamp, ctx->ws.lru_order,
                     ctx->ws.tok2slot, ctx->lay.lmax, ctx->ws.req_step, ctx->ws.req_used,
                     ctx->ws.win_start, ctx->ws.guess, ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_HOT_RELEASE, false, stream);
  return hipGetLastError();
}

hipError_t hs_launch_pool_give(const hs_ctx* ctx, const int32_t* blocks, int n, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  hs_timer_mark(ctx, HS_KERNEL_POOL_GIVE, true, stream);
  hipLaunchKernelGGL(pool_append_kernel, dim3(1), dim3(64), 0, stream, blocks, n, 0, c.max_batch,
                     ctx->lay.hot_rows / kBlock, ctx->buf.hot_blocks, ctx->ws.pool_ring,
                     ctx->ws.pool_ctr, (int64_t)c.num_gpu_blocks, (int64_t)c.num_gpu_blocks,
                     ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_POOL_GIVE, false, stream);
  return hipGetLastError();
}

hipError_t hs_launch_hot_reset(const hs_ctx* ctx, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  const int64_t n_slots = (int64_t)c.max_batch * ctx->lay.hot_rows;
  const int64_t n_tok = (int64_t)c.max_batch * ctx->lay.lmax;
  const int64_t n_hot_blocks = c.hot_leasing ? (int64_t)c.max_batch * (ctx->lay.hot_rows / kBlock) : 0;
  int64_t n = n_tok;
  if (n_slots > n) n = n_slots;
  if (n_hot_blocks > n) n = n_hot_blocks;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hs_timer_mark(ctx, HS_KERNEL_HOT_RESET, true, stream);
  hipLaunchKernelGGL(hot_reset_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     ctx->ws.slot_token, ctx->ws.slot_stamp, ctx->ws.lru_order, n_slots,
                     ctx->lay.hot_rows, ctx->ws.tok2slot, n_tok, ctx->ws.req_step, ctx->ws.req_used,
                     ctx->ws.win_start, c.max_batch, ctx->ws.guess,
                     c.max_batch * c.max_queries, ctx->ws.path_count, ctx->buf.hot_blocks,
                     n_hot_blocks, c.hot_leasing ? ctx->ws.pool_ctr : nullptr, n, ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_HOT_RESET, false, stream);
  return hipGetLastError();
}

// The resolver's dynamic-LDS limit: everything a CU's 160 KiB leaves beside the kernel's static
// arrays.  The attribute is process-wide (per kernel, not per context), so it is always set to
// this one maximum: a context created later can never lower it under a live one, and every
// layout a call picks (at most 160 KiB less 2 KiB) stays within it.
hipError_t hs_resolve_set_attributes() {
  hipFuncAttributes fa;
  hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&resolve_kernel));
  if (e != hipSuccess) return e;
  const int lds = 160 * 1024 - (int)fa.sharedSizeBytes;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&resolve_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
}
