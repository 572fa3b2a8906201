// C ABI of the HiSparse decode-step library: argument checks, workspace layout, the pinned
// host pool, and kernel launches.  No call here allocates device memory; the step calls
// (index_topk, resolve, decode) never synchronise.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "hisparse.h"
#include "hs_internal.h"

namespace hs {

struct KernelTimer {
  static constexpr size_t kEvents = 16384;
  struct Rec {
    int kernel;
    hipEvent_t begin, end;
  };
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  std::vector<Rec> recs;
  bool overflow = false;
  bool open = false;  // a begin mark waits for its end mark
};

}  // namespace hs

void hs_timer_mark(const hs_ctx* ctx, int kernel, bool begin, hipStream_t stream) {
  hs::KernelTimer* t = ctx->timer;
  if (!t) return;
  if (begin) {
    t->open = false;
    if (t->next + 2 > t->pool.size()) {
      t->overflow = true;
      return;
    }
    hipEvent_t a = t->pool[t->next++];
    if (hipEventRecord(a, stream) != hipSuccess) {
      t->overflow = true;
      return;
    }
    t->recs.push_back({kernel, a, nullptr});
    t->open = true;
  } else if (t->open) {
    t->open = false;
    hipEvent_t b = t->pool[t->next++];
    if (hipEventRecord(b, stream) != hipSuccess) {
      t->recs.pop_back();
      t->overflow = true;
      return;
    }
    t->recs.back().end = b;
  }
}

static void timer_free(hs_ctx* ctx) {
  if (!ctx->timer) return;
  for (hipEvent_t e : ctx->timer->pool) (void)hipEventDestroy(e);
  delete ctx->timer;
  ctx->timer = nullptr;
}

hipError_t hs_set_kernel_attributes();
hipError_t hs_resolve_set_attributes();
hipError_t hs_select_set_attributes();

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hs_status fail(hs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hs_status ok() {
  g_last_error.clear();
  return HS_OK;
}

hs_status hip_fail(hipError_t e, const char* what) {
  return fail(HS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int default_hot_rows(const hs_config& c) {
  const int64_t want = (int64_t)(c.max_queries + 1) * c.topk;
  return (int)((want + hs::kBlock - 1) / hs::kBlock * hs::kBlock);
}

hs_status validate(const hs_config* c) {
  if (!c) return fail(HS_ERR_INVALID_ARG, "config is NULL");
  if (c->block_size != hs::kBlock) return fail(HS_ERR_UNSUPPORTED, "block_size must be 64");
  if (c->n_idx_heads != hs::kIdxHeads || c->idx_dim != hs::kIdxDim)
    return fail(HS_ERR_UNSUPPORTED, "indexer shape must be 32 heads x 128 dims");
  if (c->n_heads != hs::kHeads || c->d_qk != hs::kDqk || c->d_v != hs::kDv)
    return fail(HS_ERR_UNSUPPORTED, "MLA shape must be 64 heads, d_qk 576, d_v 512");
  if ((c->kv_dtype != HS_BF16 && c->kv_dtype != HS_FP8_E4M3) ||
      (c->idx_dtype != HS_BF16 && c->idx_dtype != HS_FP8_E4M3))
    return fail(HS_ERR_UNSUPPORTED, "dtype must be HS_BF16 or HS_FP8_E4M3");
  if (c->topk < 1 || c->topk > hs::kMaxTopk) return fail(HS_ERR_UNSUPPORTED, "topk must be in [1, 2048]");
  if (c->n_layers < 1 || c->n_layers > 16) return fail(HS_ERR_INVALID_ARG, "n_layers must be in [1, 16]");
  if (c->max_batch < 1) return fail(HS_ERR_INVALID_ARG, "max_batch must be >= 1");
  if (c->max_queries < 1 || c->max_queries > hs::kMaxQueries)
    return fail(HS_ERR_UNSUPPORTED, "max_queries must be in [1, 4]");
  if (c->max_pages_per_req < 1 || (int64_t)c->max_pages_per_req * hs::kBlock > (1ll << 30))
    return fail(HS_ERR_INVALID_ARG, "max_pages_per_req out of range");
  // the sweep addresses one request's score rows (S x tokens x 4 bytes) with 31-bit offsets
  if ((int64_t)c->max_queries * c->max_pages_per_req * hs::kBlock * 4 >= (1ll << 31))
    return fail(HS_ERR_INVALID_ARG, "max_queries x max_pages_per_req too large (score rows over 2 GiB)");
  const int H = c->hot_rows_per_req ? c->hot_rows_per_req : default_hot_rows(*c);
  if (H % hs::kBlock != 0 || H > hs::kMaxHot)
    return fail(HS_ERR_INVALID_ARG, "hot_rows_per_req must be a multiple of 64 and <= 16384 (got %d)", H);
  if (H < c->max_queries * c->topk)
    return fail(HS_ERR_INVALID_ARG,
                "hot buffer of %d rows cannot hold the %d x %d rows one call may select", H,
                c->max_queries, c->topk);
  if (c->topk_lds_candidates < 0) return fail(HS_ERR_INVALID_ARG, "topk_lds_candidates must be >= 0");
  if (c->num_gpu_blocks < 1 || c->num_gpu_blocks * hs::kBlock > INT32_MAX)
    return fail(HS_ERR_INVALID_ARG, "num_gpu_blocks out of range (row ids are int32)");
  if (c->num_idx_blocks < 1 || c->num_idx_blocks > INT32_MAX)
    return fail(HS_ERR_INVALID_ARG, "num_idx_blocks out of range");
  if (c->num_host_blocks < 0 || c->num_host_blocks * hs::kBlock > INT32_MAX)
    return fail(HS_ERR_INVALID_ARG, "num_host_blocks out of range (host rows are int32)");
  if (c->hot_leasing != 0 && c->hot_leasing != 1)
    return fail(HS_ERR_INVALID_ARG, "hot_leasing must be 0 or 1");
  if (c->hot_leasing && c->num_host_blocks == 0)
    return fail(HS_ERR_INVALID_ARG, "hot_leasing needs a host pool (num_host_blocks > 0)");
  return HS_OK;
}

}  // namespace

hs_status hs::compute_layout(const hs_config& c, Layout* L) {
  const int64_t B = c.max_batch, S = c.max_queries;
  L->hot_rows = c.hot_rows_per_req ? c.hot_rows_per_req : default_hot_rows(c);
  L->lmax = (int64_t)c.max_pages_per_req * kBlock;
  L->bm_words = (L->lmax + 1023) / 1024 * 32;
  int64_t cap = (1024 + B * S - 1) / (B * S);
  if (cap < 2) cap = 2;
  if (cap > kMaxSplits) cap = kMaxSplits;
  L->splits_cap = (int32_t)cap;
  const int64_t H = L->hot_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L->off_slot_token = take(B * H * 4);
  L->off_slot_stamp = take(B * H * 4);
  L->off_lru_order = take(2 * B * H * 4);
  L->off_tok2slot = take(B * L->lmax * 4);
  L->off_req_step = take(B * 4);
  L->off_req_used = take(B * 4);
  L->off_win_start = take(B * 4);
  L->off_pool_ring = take((size_t)c.num_gpu_blocks * 4);
  L->off_pool_ctr = take(2 * 8);
  L->off_err = take(4);
  L->off_scores = take(B * S * L->lmax * 4);
  L->off_bitmap = take(B * S * L->bm_words * 4);
  L->off_miss_src = take(B * S * c.topk * 4);
  L->off_miss_dst = take(B * S * c.topk * 4);
  L->off_miss_cnt = take(B * 4);
  L->off_part_o = take(B * S * cap * kHeads * kDv * 4);
  L->off_part_ml = take(B * S * cap * kHeads * 2 * 4);
  L->n_seg = (int32_t)((c.max_pages_per_req + kPagesPerItem - 1) / kPagesPerItem * kSweepWaves);
  L->off_guess = take(B * S * 4);
  L->off_rescore = take((B * S + 1) * 4);
  L->off_seg_count = take(B * S * L->n_seg * 4);
  L->off_cands = take(B * S * L->n_seg * kSegCap * 8);
  L->off_path_count = take(2 * 8);
  L->off_zero_row = take(kZeroRowBytes);
  L->off_pf_lens = take(B * 4);
  L->off_pf_guess = take(B * S * 4);
  L->off_pf_paths = take(2 * 8);
  L->off_pf_rows = take(B * S * c.topk * 4);
  L->total = off;
  return HS_OK;
}

extern "C" {

hs_status hs_kernel_timing(hs_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "ctx is NULL");
  if (!enable) {
    timer_free(ctx);
    return ok();
  }
  if (ctx->timer) return ok();
  hipError_t e = hipSetDevice(ctx->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  auto* t = new hs::KernelTimer();
  t->pool.reserve(hs::KernelTimer::kEvents);
  for (size_t i = 0; i < hs::KernelTimer::kEvents; ++i) {
    hipEvent_t ev;
    e = hipEventCreate(&ev);
    if (e != hipSuccess) break;
    t->pool.push_back(ev);
  }
  ctx->timer = t;
  if (e != hipSuccess) {
    timer_free(ctx);
    return hip_fail(e, "hipEventCreate");
  }
  return ok();
}

hs_status hs_kernel_times(hs_ctx* ctx, double* ms, int64_t* launches, int32_t n) {
  if (!ctx || !ms || !launches || n < 0) return fail(HS_ERR_INVALID_ARG, "bad argument");
  if (!ctx->timer) return fail(HS_ERR_STATE, "kernel timing is not enabled");
  hs::KernelTimer* t = ctx->timer;
  for (int32_t i = 0; i < n; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  hipError_t e = hipSuccess;
  for (const auto& r : t->recs) {
    if (!r.end) continue;
    e = hipEventSynchronize(r.end);
    if (e != hipSuccess) break;
    float v = 0.0f;
    e = hipEventElapsedTime(&v, r.begin, r.end);
    if (e != hipSuccess) break;
    if (r.kernel >= 0 && r.kernel < n) {
      ms[r.kernel] += v;
      launches[r.kernel] += 1;
    }
  }
  const bool overflow = t->overflow;
  t->recs.clear();
  t->next = 0;
  t->overflow = false;
  t->open = false;
  if (e != hipSuccess) return hip_fail(e, "hs_kernel_times");
  if (overflow) return fail(HS_ERR_STATE, "event pool exhausted: some launches were not timed");
  return ok();
}

const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "HS_OK";
    case HS_ERR_INVALID_ARG: return "HS_ERR_INVALID_ARG";
    case HS_ERR_UNSUPPORTED: return "HS_ERR_UNSUPPORTED";
    case HS_ERR_OUT_OF_MEMORY: return "HS_ERR_OUT_OF_MEMORY";
    case HS_ERR_HIP: return "HS_ERR_HIP";
    case HS_ERR_STATE: return "HS_ERR_STATE";
  }
  return "unknown hs_status";
}

const char* hs_last_error(void) { return g_last_error.c_str(); }

hs_status hs_workspace_bytes(const hs_config* cfg, size_t* dev_bytes) {
  hs_status s = validate(cfg);
  if (s != HS_OK) return s;
  if (!dev_bytes) return fail(HS_ERR_INVALID_ARG, "dev_bytes is NULL");
  hs::Layout L;
  hs::compute_layout(*cfg, &L);
  *dev_bytes = L.total;
  return ok();
}

hs_status hs_host_pool_bytes(const hs_config* cfg, size_t* host_bytes) {
  hs_status s = validate(cfg);
  if (s != HS_OK) return s;
  if (!host_bytes) return fail(HS_ERR_INVALID_ARG, "host_bytes is NULL");
  const size_t rb = cfg->kv_dtype == HS_FP8_E4M3 ? hs::kFp8Row : hs::kBf16Row;
  *host_bytes = (size_t)cfg->n_layers * (size_t)cfg->num_host_blocks * hs::kBlock * rb;
  return ok();
}

hs_status hs_create(const hs_config* cfg, hs_ctx** out) {
  hs_status s = validate(cfg);
  if (s != HS_OK) return s;
  if (!out) return fail(HS_ERR_INVALID_ARG, "out is NULL");
  hs_ctx* ctx = new hs_ctx();
  ctx->cfg = *cfg;
  hs::compute_layout(*cfg, &ctx->lay);
  ctx->row_bytes = cfg->kv_dtype == HS_FP8_E4M3 ? hs::kFp8Row : hs::kBf16Row;
  ctx->idx_block_bytes = cfg->idx_dtype == HS_FP8_E4M3 ? hs::kIdxFp8Block : hs::kIdxBf16Block;
  ctx->host_pool = nullptr;
  ctx->host_pool_dev = nullptr;
  ctx->host_pool_bytes = 0;
  ctx->bound = false;
  std::memset(&ctx->buf, 0, sizeof(ctx->buf));
  std::memset(&ctx->ws, 0, sizeof(ctx->ws));
  hipError_t e = hipGetDevice(&ctx->device);
  if (e == hipSuccess) e = hs_set_kernel_attributes();
  if (e == hipSuccess) e = hs_resolve_set_attributes();
  if (e == hipSuccess) e = hs_select_set_attributes();
  if (e == hipSuccess) e = hs_fixed_scratch_init(ctx->device);
  if (e != hipSuccess) {
    delete ctx;
    return hip_fail(e, "hs_create");
  }
  *out = ctx;
  return ok();
}

hs_status hs_destroy(hs_ctx* ctx) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "ctx is NULL");
  timer_free(ctx);
  if (ctx->host_pool) (void)hipHostFree(ctx->host_pool);
  delete ctx;
  return ok();
}

hs_status hs_host_pool_alloc(hs_ctx* ctx, void** host_base) {
  if (!ctx || !host_base) return fail(HS_ERR_INVALID_ARG, "ctx or host_base is NULL");
  if (ctx->host_pool) return fail(HS_ERR_STATE, "host pool already allocated");
  size_t bytes = 0;
  hs_host_pool_bytes(&ctx->cfg, &bytes);
  *host_base = nullptr;
  if (bytes == 0) return ok();
  hipError_t e = hipSetDevice(ctx->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  void* p = nullptr;
  e = hipHostMalloc(&p, bytes, hipHostMallocMapped);
  if (e != hipSuccess || !p)
    return fail(HS_ERR_OUT_OF_MEMORY, "hipHostMalloc(%zu bytes, mapped): %s", bytes, hipGetErrorString(e));
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, p, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(p);
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  ctx->host_pool = p;
  ctx->host_pool_dev = d;
  ctx->host_pool_bytes = bytes;
  *host_base = p;
  return ok();
}

hs_status hs_bind(hs_ctx* ctx, const hs_buffers* b) {
  if (!ctx || !b) return fail(HS_ERR_INVALID_ARG, "ctx or buffers is NULL");
  if (!b->kv_pool || !b->idx_pool || !b->idx_block_table || !b->block_table ||
      !b->host_block_table || !b->hot_blocks || !b->workspace)
    return fail(HS_ERR_INVALID_ARG, "a bound buffer is NULL");
  if (reinterpret_cast<uintptr_t>(b->workspace) % 256 != 0)
    return fail(HS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (reinterpret_cast<uintptr_t>(b->kv_pool) % 16 != 0 || reinterpret_cast<uintptr_t>(b->idx_pool) % 16 != 0)
    return fail(HS_ERR_INVALID_ARG, "kv_pool and idx_pool must be 16-byte aligned");
  if (ctx->cfg.num_host_blocks > 0 && !ctx->host_pool)
    return fail(HS_ERR_STATE, "allocate the host pool (hs_host_pool_alloc) before binding");
  ctx->buf = *b;
  unsigned char* w = static_cast<unsigned char*>(b->workspace);
  const hs::Layout& L = ctx->lay;
  ctx->ws.slot_token = reinterpret_cast<int32_t*>(w + L.off_slot_token);
  ctx->ws.slot_stamp = reinterpret_cast<int32_t*>(w + L.off_slot_stamp);
  ctx->ws.lru_order = reinterpret_cast<int32_t*>(w + L.off_lru_order);
  ctx->ws.tok2slot = reinterpret_cast<int32_t*>(w + L.off_tok2slot);
  ctx->ws.req_step = reinterpret_cast<int32_t*>(w + L.off_req_step);
  ctx->ws.req_used = reinterpret_cast<int32_t*>(w + L.off_req_used);
  ctx->ws.win_start = reinterpret_cast<int32_t*>(w + L.off_win_start);
  ctx->ws.pool_ring = reinterpret_cast<int32_t*>(w + L.off_pool_ring);
  ctx->ws.pool_ctr = reinterpret_cast<int64_t*>(w + L.off_pool_ctr);
  ctx->ws.err = reinterpret_cast<int32_t*>(w + L.off_err);
  ctx->ws.scores = reinterpret_cast<float*>(w + L.off_scores);
  ctx->ws.bitmap = reinterpret_cast<uint32_t*>(w + L.off_bitmap);
  ctx->ws.miss_src = reinterpret_cast<int32_t*>(w + L.off_miss_src);
  ctx->ws.miss_dst = reinterpret_cast<int32_t*>(w + L.off_miss_dst);
  ctx->ws.miss_cnt = reinterpret_cast<int32_t*>(w + L.off_miss_cnt);
  ctx->ws.part_o = reinterpret_cast<float*>(w + L.off_part_o);
  ctx->ws.part_ml = reinterpret_cast<float*>(w + L.off_part_ml);
  ctx->ws.guess = reinterpret_cast<uint32_t*>(w + L.off_guess);
  ctx->ws.rescore = reinterpret_cast<int32_t*>(w + L.off_rescore);
  ctx->ws.n_rescore = ctx->ws.rescore + (int64_t)ctx->cfg.max_batch * ctx->cfg.max_queries;
  ctx->ws.seg_count = reinterpret_cast<uint32_t*>(w + L.off_seg_count);
  ctx->ws.cands = reinterpret_cast<uint64_t*>(w + L.off_cands);
  ctx->ws.path_count = reinterpret_cast<unsigned long long*>(w + L.off_path_count);
  ctx->ws.zero_row = w + L.off_zero_row;
  ctx->ws.pf_lens = reinterpret_cast<int32_t*>(w + L.off_pf_lens);
  ctx->ws.pf_guess = reinterpret_cast<uint32_t*>(w + L.off_pf_guess);
  ctx->ws.pf_paths = reinterpret_cast<unsigned long long*>(w + L.off_pf_paths);
  ctx->ws.pf_rows = reinterpret_cast<int32_t*>(w + L.off_pf_rows);
  // the row of zeros the decode reads for skipped rows: written once here, read-only for
  // every kernel
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipMemset(ctx->ws.zero_row, 0, hs::kZeroRowBytes);
  if (e != hipSuccess) return hip_fail(e, "hs_bind: clearing the zero row");
  ctx->bound = true;
  return ok();
}

hs_status hs_hot_reset(hs_ctx* ctx, void* stream) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "ctx is NULL");
  if (!ctx->bound) return fail(HS_ERR_STATE, "context is not bound");
  hipError_t e = hs_launch_hot_reset(ctx, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hot reset launch");
}

static hs_status check_step(const hs_ctx* ctx, int32_t B, int32_t S, const char* what) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "%s: ctx is NULL", what);
  if (!ctx->bound) return fail(HS_ERR_STATE, "%s: context is not bound", what);
  if (B < 0 || B > ctx->cfg.max_batch)
    return fail(HS_ERR_INVALID_ARG, "%s: B=%d outside [0, %d]", what, B, ctx->cfg.max_batch);
  if (S < 1 || S > ctx->cfg.max_queries)
    return fail(HS_ERR_INVALID_ARG, "%s: S=%d outside [1, %d]", what, S, ctx->cfg.max_queries);
  return HS_OK;
}

hs_status hisparse_index_topk(hs_ctx* ctx, const void* q_idx, const float* w,
                              const int32_t* ctx_lens, int32_t B, int32_t S, int32_t* topk_out,
                              void* stream) {
  hs_status s = check_step(ctx, B, S, "hisparse_index_topk");
  if (s != HS_OK) return s;
  if (B == 0) return ok();
  if (!q_idx || !w || !ctx_lens || !topk_out)
    return fail(HS_ERR_INVALID_ARG, "hisparse_index_topk: a pointer argument is NULL");
  hipError_t e = hs_launch_index_topk(ctx, q_idx, w, ctx_lens, B, S, topk_out,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hisparse_index_topk launch");
}

hs_status hisparse_resolve_plan(hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens,
                                int32_t B, int32_t S, const int32_t* begin_window,
                                int32_t* row_ids_out, int32_t* stats_out, void* stream) {
  hs_status s = check_step(ctx, B, S, "hisparse_resolve");
  if (s != HS_OK) return s;
  if (B == 0) return ok();
  if (!topk || !ctx_lens || !row_ids_out)
    return fail(HS_ERR_INVALID_ARG, "hisparse_resolve: a pointer argument is NULL");
  if (ctx->cfg.num_host_blocks > 0 && !ctx->host_pool_dev)
    return fail(HS_ERR_STATE, "hisparse_resolve: host pool missing");
  hipError_t e = hs_launch_resolve(ctx, topk, ctx_lens, B, S, begin_window, row_ids_out,
                                   stats_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hisparse_resolve launch");
}

hs_status hisparse_resolve(hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens, int32_t B,
                           int32_t S, int32_t* row_ids_out, int32_t* stats_out, void* stream) {
  return hisparse_resolve_plan(ctx, topk, ctx_lens, B, S, nullptr, row_ids_out, stats_out, stream);
}

static hs_status check_list(const hs_ctx* ctx, const int32_t* list, int32_t n, const char* what) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "%s: ctx is NULL", what);
  if (!ctx->bound) return fail(HS_ERR_STATE, "%s: context is not bound", what);
  if (n < 0) return fail(HS_ERR_INVALID_ARG, "%s: n=%d is negative", what, n);
  if (n > 0 && !list) return fail(HS_ERR_INVALID_ARG, "%s: list is NULL", what);
  return HS_OK;
}

hs_status hs_hot_release(hs_ctx* ctx, const int32_t* reqs, int32_t n, void* stream) {
  hs_status s = check_list(ctx, reqs, n, "hs_hot_release");
  if (s != HS_OK || n == 0) return s;
  hipError_t e = hs_launch_hot_release(ctx, reqs, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hs_hot_release launch");
}

hs_status hs_hot_pool_give(hs_ctx* ctx, const int32_t* blocks, int32_t n, void* stream) {
  hs_status s = check_list(ctx, blocks, n, "hs_hot_pool_give");
  if (s != HS_OK) return s;
  if (!ctx->cfg.hot_leasing) return fail(HS_ERR_STATE, "hs_hot_pool_give: the context does not lease hot pages");
  if (n == 0) return ok();
  hipError_t e = hs_launch_pool_give(ctx, blocks, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hs_hot_pool_give launch");
}

hs_status hs_hot_pool_read(hs_ctx* ctx, int32_t* out, int32_t cap, int32_t* n) {
  if (!ctx || !n || cap < 0 || (cap > 0 && !out)) return fail(HS_ERR_INVALID_ARG, "hs_hot_pool_read: bad argument");
  if (!ctx->bound) return fail(HS_ERR_STATE, "hs_hot_pool_read: context is not bound");
  if (!ctx->cfg.hot_leasing) return fail(HS_ERR_STATE, "hs_hot_pool_read: the context does not lease hot pages");
  int64_t ctr[2] = {0, 0};
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(ctr, ctx->ws.pool_ctr, sizeof(ctr), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hs_hot_pool_read");
  const int64_t ring = ctx->cfg.num_gpu_blocks;
  const int64_t count = ctr[1] - ctr[0];
  if (count < 0 || count > ring) return fail(HS_ERR_STATE, "hs_hot_pool_read: pool counters corrupt");
  std::vector<int32_t> all((size_t)ring);
  e = hipMemcpy(all.data(), ctx->ws.pool_ring, (size_t)ring * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hs_hot_pool_read");
  for (int64_t i = 0; i < count && i < cap; ++i) out[i] = all[(size_t)((ctr[0] + i) % ring)];
  *n = (int32_t)count;
  return ok();
}

hs_status sparse_mla_decode(hs_ctx* ctx, int32_t layer, const void* q, const int32_t* row_ids,
                            const int32_t* ctx_lens, int32_t B, int32_t S, float sm_scale,
                            void* out, float* lse, void* stream) {
  hs_status s = check_step(ctx, B, S, "sparse_mla_decode");
  if (s != HS_OK) return s;
  if (layer < 0 || layer >= ctx->cfg.n_layers)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode: layer %d outside [0, %d)", layer, ctx->cfg.n_layers);
  if (!std::isfinite(sm_scale)) return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode: sm_scale not finite");
  if (B == 0) return ok();
  if (!q || !row_ids || !ctx_lens || !out)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode: a pointer argument is NULL");
  const int splits = hs_choose_splits(ctx, B, S);
  hipError_t e = hs_launch_decode(ctx, layer, q, row_ids, ctx_lens, B, S, sm_scale, out, lse,
                                  splits, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "sparse_mla_decode launch");
}

static hs_status check_prefill(const hs_ctx* ctx, int32_t b, int32_t L, int32_t P, const char* what) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "%s: ctx is NULL", what);
  if (!ctx->bound) return fail(HS_ERR_STATE, "%s: context is not bound", what);
  if (b < 0 || b >= ctx->cfg.max_batch)
    return fail(HS_ERR_INVALID_ARG, "%s: request %d outside [0, %d)", what, b, ctx->cfg.max_batch);
  if (P < 1 || L < P || (int64_t)L > (int64_t)ctx->cfg.max_pages_per_req * hs::kBlock)
    return fail(HS_ERR_INVALID_ARG, "%s: need 1 <= P <= L <= %lld (P=%d, L=%d)", what,
                (long long)ctx->cfg.max_pages_per_req * hs::kBlock, P, L);
  return HS_OK;
}

hs_status hisparse_prefill_index_topk(hs_ctx* ctx, int32_t b, const void* q_idx, const float* w,
                                      int32_t L, int32_t P, int32_t* topk_out, void* stream) {
  hs_status s = check_prefill(ctx, b, L, P, "hisparse_prefill_index_topk");
  if (s != HS_OK) return s;
  if (!q_idx || !w || !topk_out)
    return fail(HS_ERR_INVALID_ARG, "hisparse_prefill_index_topk: a pointer argument is NULL");
  hipError_t e = hs_launch_prefill_index_topk(ctx, b, q_idx, w, L, P, topk_out,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hisparse_prefill_index_topk launch");
}

hs_status sparse_mla_prefill(hs_ctx* ctx, int32_t layer, int32_t b, const void* q,
                             const int32_t* topk, int32_t L, int32_t P, float sm_scale, void* out,
                             float* lse, void* stream) {
  hs_status s = check_prefill(ctx, b, L, P, "sparse_mla_prefill");
  if (s != HS_OK) return s;
  if (layer < 0 || layer >= ctx->cfg.n_layers)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_prefill: layer %d outside [0, %d)", layer, ctx->cfg.n_layers);
  if (!std::isfinite(sm_scale)) return fail(HS_ERR_INVALID_ARG, "sparse_mla_prefill: sm_scale not finite");
  if (!q || !out) return fail(HS_ERR_INVALID_ARG, "sparse_mla_prefill: a pointer argument is NULL");
  if (!topk && L > ctx->cfg.topk)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_prefill: without a top-K the context (%d) must fit top-K (%d)",
                L, ctx->cfg.topk);
  hipError_t e = hs_launch_prefill_decode(ctx, layer, b, q, topk, L, P, sm_scale, out, lse,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "sparse_mla_prefill launch");
}

hs_status sparse_mla_decode_noalloc(hs_ctx* ctx, int32_t layer, const void* q,
                                    const int32_t* row_ids, const int32_t* ctx_lens, int32_t B,
                                    int32_t S, float sm_scale, void* out, float* lse, void* stream) {
  hs_status s = check_step(ctx, B, S, "sparse_mla_decode_noalloc");
  if (s != HS_OK) return s;
  if (layer < 0 || layer >= ctx->cfg.n_layers)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode_noalloc: layer %d outside [0, %d)", layer,
                ctx->cfg.n_layers);
  if (!std::isfinite(sm_scale)) return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode_noalloc: sm_scale not finite");
  if (B == 0) return ok();
  if (!q || !row_ids || !ctx_lens || !out)
    return fail(HS_ERR_INVALID_ARG, "sparse_mla_decode_noalloc: a pointer argument is NULL");
  const int splits = hs_choose_splits(ctx, B, S);
  const int64_t partials = splits > 1 ? (int64_t)B * S * splits : 0;
  if (partials > hs::kFixedPartials)
    return fail(HS_ERR_INVALID_ARG,
                "sparse_mla_decode_noalloc: %d queries x %d splits need %lld split partials; the "
                "fixed scratch holds %d", B * S, splits, (long long)partials, hs::kFixedPartials);
  unsigned char* p = static_cast<unsigned char*>(hs_fixed_scratch(ctx->device));
  if (!p) return fail(HS_ERR_STATE, "sparse_mla_decode_noalloc: no fixed scratch on device %d", ctx->device);
  float* part_o = reinterpret_cast<float*>(p);
  float* part_ml = reinterpret_cast<float*>(p + (size_t)hs::kFixedPartials * hs::kHeads * hs::kDv * 4);
  hipError_t e = hs_launch_decode(ctx, layer, q, row_ids, ctx_lens, B, S, sm_scale, out, lse,
                                  splits, static_cast<hipStream_t>(stream), part_o, part_ml);
  return e == hipSuccess ? ok() : hip_fail(e, "sparse_mla_decode_noalloc launch");
}

hs_status hs_decode_splits(const hs_ctx* ctx, int32_t B, int32_t S, int32_t* splits) {
  if (!ctx || !splits) return fail(HS_ERR_INVALID_ARG, "ctx or splits is NULL");
  if (B < 1 || S < 1) return fail(HS_ERR_INVALID_ARG, "B and S must be >= 1");
  *splits = hs_choose_splits(ctx, B, S);
  return ok();
}

hs_status hs_hot_state(const hs_ctx* ctx, hs_hot_state_ptrs* out) {
  if (!ctx || !out) return fail(HS_ERR_INVALID_ARG, "ctx or out is NULL");
  if (!ctx->bound) return fail(HS_ERR_STATE, "context is not bound");
  out->slot_token = ctx->ws.slot_token;
  out->slot_stamp = ctx->ws.slot_stamp;
  out->tok2slot = ctx->ws.tok2slot;
  out->req_step = ctx->ws.req_step;
  out->hot_rows = ctx->lay.hot_rows;
  out->reserved = 0;
  out->tokens_per_req = ctx->lay.lmax;
  return ok();
}

hs_status hs_read_device_error(hs_ctx* ctx, int32_t* code) {
  if (!ctx || !code) return fail(HS_ERR_INVALID_ARG, "ctx or code is NULL");
  if (!ctx->bound) return fail(HS_ERR_STATE, "context is not bound");
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(code, ctx->ws.err, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    const int32_t zero = 0;
    e = hipMemcpy(ctx->ws.err, &zero, 4, hipMemcpyHostToDevice);
  }
  return e == hipSuccess ? ok() : hip_fail(e, "hs_read_device_error");
}

static hs_status check_pages(const hs_ctx* ctx, const int32_t* pages, int32_t n, const char* what) {
  if (!ctx) return fail(HS_ERR_INVALID_ARG, "%s: ctx is NULL", what);
  if (!ctx->bound) return fail(HS_ERR_STATE, "%s: context is not bound", what);
  if (n < 0) return fail(HS_ERR_INVALID_ARG, "%s: n=%d is negative", what, n);
  if (n > 0 && !pages) return fail(HS_ERR_INVALID_ARG, "%s: pages is NULL", what);
  if (n > 0 && (ctx->cfg.num_host_blocks == 0 || !ctx->host_pool_dev))
    return fail(HS_ERR_STATE, "%s: no host pool", what);
  return HS_OK;
}

hs_status hisparse_materialize_pages(hs_ctx* ctx, const int32_t* pages, int32_t n, void* stream) {
  hs_status s = check_pages(ctx, pages, n, "hisparse_materialize_pages");
  if (s != HS_OK || n == 0) return s;
  hipError_t e = hs_launch_materialize(ctx, pages, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hisparse_materialize_pages launch");
}

hs_status hisparse_release_pages(hs_ctx* ctx, const int32_t* pages, int32_t n,
                                 const int32_t* ctx_lens, int32_t* freed_out, void* stream) {
  hs_status s = check_pages(ctx, pages, n, "hisparse_release_pages");
  if (s != HS_OK || n == 0) return s;
  if (!ctx_lens || !freed_out)
    return fail(HS_ERR_INVALID_ARG, "hisparse_release_pages: ctx_lens or freed_out is NULL");
  hipError_t e = hs_launch_release(ctx, pages, n, ctx_lens, freed_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "hisparse_release_pages launch");
}

hs_status hs_select_paths(hs_ctx* ctx, int64_t* from_candidates, int64_t* from_scores) {
  if (!ctx || !from_candidates || !from_scores) return fail(HS_ERR_INVALID_ARG, "NULL argument");
  if (!ctx->bound) return fail(HS_ERR_STATE, "context is not bound");
  unsigned long long v[2] = {0, 0};
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(v, ctx->ws.path_count, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hs_select_paths");
  *from_candidates = (int64_t)v[0];
  *from_scores = (int64_t)v[1];
  return ok();
}

}  // extern "C"
