/*
 * hisparse.h -- C ABI of the Hybrid HiSparse sparse-MLA decode step on MI355X (gfx950).
 *
 * One decode step of sparse MLA with the KV of old pages offloaded to pinned host memory:
 *
 *   hisparse_index_topk  the indexer scores every earlier token of each request and keeps
 *                        the top-K (2,048) of them.  GLM-5.3 part-2 page, "Why not TP or
 *                        DP?" (the indexer scores every earlier token and picks the 2,048
 *                        that sparse MLA attends to); Hybrid HiSparse part-1 page, "Using
 *                        sparsity when it is needed" (the indexer picks the top-K tokens,
 *                        indexer keys stay on the GPU).
 *   hisparse_resolve     the fused top-K resolver: each selected token is read in place
 *                        when its page is GPU-resident, read from the hot buffer (and its
 *                        LRU entry refreshed) when it is hot, or copied as a single row from
 *                        pinned host memory into an LRU victim slot when it is a miss.  It
 *                        emits row ids into one shared paged KV tensor, gathered with one
 *                        stride.  Part-1 page, "How it works" (hybrid residency bullet; the
 *                        paragraph on hot-buffer pages leased from the shared pool).
 *   sparse_mla_decode    sparse MLA decode attention (MQA form): all 64 heads share one
 *                        576-dim latent row (512 "nope" + 64 rope) as key, and its first 512
 *                        dims as value.  Part-2 page, "Try it" (the sparse-MLA MQA kernel)
 *                        and footnote 1 (656-byte FP8 rows, QK over 576 dims, PV over 512).
 *
 * Around the step: the write side of the host pool (hisparse_materialize_pages,
 * hisparse_release_pages), hot pages leased from a free-block pool and released per request
 * (hs_config.hot_leasing, hs_hot_pool_give, hs_hot_release), plan windows for speculative
 * decoding (hisparse_resolve_plan), and the prefill of a prompt on the same kernels
 * (hisparse_prefill_index_topk, sparse_mla_prefill).
 *
 * Conventions shared by every call:
 *   - Status codes are returned; nothing throws across the ABI.  hs_last_error() gives a
 *     human-readable reason for the last failing call on the calling thread.
 *   - Arguments are checked on the host without synchronising.  Faults only the device can
 *     see (a placeholder page without a host copy, a block or row id out of range, a
 *     context shorter than its query count) set a sticky device error word, read with
 *     hs_read_device_error() outside the hot loop; the offending item is skipped, no access
 *     leaves its buffer, and the other results of that call are unspecified (a skipped key
 *     page leaves its tokens' scores stale; a skipped row id, or -1 inside a query's range,
 *     is left out of that query's softmax).
 *   - Device buffers are borrowed: the caller allocates them (e.g. with PyTorch) and keeps
 *     them alive while bound.  The library owns only the context and the pinned host pool.
 *   - The three step calls allocate nothing, never synchronise and take every per-step
 *     value from device memory or by value, so a sequence of them can be captured into a
 *     HIP graph and replayed (part-1 page, "How it works": nothing on the decode path waits
 *     for a CPU decision).
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work of a call is enqueued
 *     on it, in order.
 *   - Block size is 64 tokens; row id = block * 64 + offset.  Shapes of the kernels are fixed:
 *     32 indexer heads x 128 dims, 64 MLA heads, d_qk = 576, d_v = 512, 1 <= S <= 4 queries.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = -1,  /* a null pointer, a size out of range, an unbound context */
  HS_ERR_UNSUPPORTED = -2,  /* a shape the kernels are not built for */
  HS_ERR_OUT_OF_MEMORY = -3,/* pinned host pool allocation failed */
  HS_ERR_HIP = -4,          /* a HIP runtime call failed (launch, device query) */
  HS_ERR_STATE = -5         /* call order violated (e.g. bind before host pool) */
} hs_status;

typedef enum { HS_BF16 = 0, HS_FP8_E4M3 = 1 } hs_dtype;

/* Device error word bits (hs_read_device_error). */
#define HS_DEVERR_NO_HOST_COPY   0x1  /* selected token on a placeholder page with no host block */
#define HS_DEVERR_BAD_BLOCK      0x2  /* block id outside its pool */
#define HS_DEVERR_BAD_ROW        0x4  /* row id outside the KV pool, or a token >= context */
#define HS_DEVERR_SHORT_CONTEXT  0x8  /* context < number of queries, or > max pages */
#define HS_DEVERR_TOPK_COUNT     0x10 /* internal: selection did not produce min(K, L) tokens */
#define HS_DEVERR_HOT_FULL       0x20 /* more misses than untouched hot slots */
#define HS_DEVERR_TAIL_PAGE      0x40 /* release of the tail page or of a page past the context */
#define HS_DEVERR_POOL_EMPTY     0x80 /* a hot page needed a block and the free-block pool was empty */
#define HS_DEVERR_POOL_FULL      0x100 /* more free blocks given than the pool holds */
#define HS_DEVERR_BAD_REQUEST    0x200 /* a request index outside [0, max_batch) */

/*
 * Static configuration.  Fixed kernel shapes must be given as listed; the rest size the
 * pools.  FP8 rows are 656 bytes: bytes [0,512) OCP E4M3 "nope" codes, [512,640) 64 bf16
 * rope values, [640,644) the fp32 scale of the nope codes, [644,656) zero (the pages give
 * only the 656-byte size).  bf16 rows are 576 bf16 values (1,152 bytes).  FP8 indexer
 * blocks hold 64 x 128 E4M3 codes then 64 fp32 scales (8,448 bytes, i.e. 132 bytes per
 * token); bf16 indexer blocks hold 64 x 128 bf16 (16,384 bytes).
 */
typedef struct hs_config {
  int32_t block_size;        /* must be 64 */
  int32_t topk;              /* K, 1..2048 (2,048 on the pages) */
  int32_t n_idx_heads;       /* must be 32 */
  int32_t idx_dim;           /* must be 128 */
  int32_t n_heads;           /* must be 64 */
  int32_t d_qk;              /* must be 576 */
  int32_t d_v;               /* must be 512 */
  int32_t kv_dtype;          /* hs_dtype of latent rows */
  int32_t idx_dtype;         /* hs_dtype of indexer keys */
  int32_t n_layers;          /* sparse-MLA layers sharing one top-K (IndexShare), 1..16 */
  int32_t max_batch;         /* B upper bound, >= 1 */
  int32_t max_queries;       /* S upper bound, 1..4 (S = 1 + speculative tokens) */
  int32_t max_pages_per_req; /* block-table width; context <= 64 * this */
  int32_t hot_rows_per_req;  /* 0 => (max_queries + 1) * topk rounded up to 64, i.e.
                                2 x top-K without MTP and (spec + 2) x top-K with MTP
                                (part-1 page: default hot buffer, and the MTP note under the
                                concurrency calculator).  Must be a multiple of 64, at least
                                max_queries * topk and at most 16384. */
  int32_t topk_lds_candidates; /* 0 => default; otherwise caps the on-chip candidate list of
                                  the top-K select (a smaller cap exercises the multi-pass
                                  path; results are identical) */
  int32_t hot_leasing;       /* 0: every request's hot pages have their blocks in hot_blocks from
                                the start.  1: hot pages are leased from the context's pool of
                                free blocks when a request first fills a slot on them and go
                                back to it when the request is released (part-1 page, "How it
                                works": hot-buffer pages are ordinary KV blocks leased from the
                                same pool as resident pages, taken when first needed and
                                returned when no longer needed; one request's freed blocks
                                become another's hot capacity).  Needs num_host_blocks > 0. */
  int64_t num_gpu_blocks;    /* blocks of the shared KV pool (resident pages + hot pages) */
  int64_t num_idx_blocks;    /* blocks of the indexer key pool */
  int64_t num_host_blocks;   /* blocks of the pinned host pool */
} hs_config;

/* Device buffers, all borrowed, all on the context's device. */
typedef struct hs_buffers {
  void* kv_pool;                   /* [n_layers][num_gpu_blocks][64][row bytes] */
  const void* idx_pool;            /* [num_idx_blocks][indexer block bytes] */
  const int32_t* idx_block_table;  /* [max_batch][max_pages_per_req] indexer block per page */
  int32_t* block_table;            /* [max_batch][max_pages_per_req] GPU block, or -1 for a
                                      placeholder whose rows live only in host memory
                                      (hisparse_release_pages writes placeholders into it) */
  const int32_t* host_block_table; /* [max_batch][max_pages_per_req] host block or -1 */
  int32_t* hot_blocks;             /* [max_batch][hot_rows/64] GPU block of each hot page.  With
                                      hot_leasing the library owns its contents: -1 for a page
                                      without a block, written by the leases and releases */
  void* workspace;                 /* hs_workspace_bytes() bytes, 256-byte aligned */
} hs_buffers;

typedef struct hs_ctx hs_ctx;

/* Validate `cfg` and create a context on the current HIP device.  No device work. */
hs_status hs_create(const hs_config* cfg, hs_ctx** out);

/* Free the pinned host pool and the context.  Bound buffers are not touched. */
hs_status hs_destroy(hs_ctx* ctx);

/* Device workspace needed by a context with this configuration: hot-buffer state
 * (slot tokens, LRU stamps and order, token-to-slot map, per-request step counters),
 * top-K scratch, split-K partials and the device error word. */
hs_status hs_workspace_bytes(const hs_config* cfg, size_t* dev_bytes);

/* Bytes of the pinned host pool: n_layers * num_host_blocks * 64 * row bytes. */
hs_status hs_host_pool_bytes(const hs_config* cfg, size_t* host_bytes);

/* Allocate the pinned, device-mapped host pool (library-owned; freed by hs_destroy) and
 * return its host address.  Layout [n_layers][num_host_blocks][64][row bytes].  The caller
 * writes host copies of placeholder pages through it.  The pool is sized in whole host
 * blocks (part-1 page, reproduction appendix: the host pool is rounded up to whole host
 * blocks).  Calling it twice returns HS_ERR_STATE. */
hs_status hs_host_pool_alloc(hs_ctx* ctx, void** host_base);

/* Bind borrowed device buffers.  Requires the host pool when num_host_blocks > 0.
 * Re-binding replaces the previous set (the hot state must then be reset). */
hs_status hs_bind(hs_ctx* ctx, const hs_buffers* bufs);

/* Reset the hot buffer of every request to cold (all slots empty, LRU clock 0, a new plan
 * window), clear the top-K scratch and the device error word.  With hot_leasing the
 * free-block pool is emptied and every hot_blocks entry set to -1 (give the pool its blocks
 * with hs_hot_pool_give afterwards).  Enqueued on `stream`. */
hs_status hs_hot_reset(hs_ctx* ctx, void* stream);

/*
 * Indexer sweep + top-K select for B requests of S query tokens each.
 *   q_idx     device [B][S][32][128] bf16 indexer queries
 *   w         device [B][S][32] fp32 non-negative head weights
 *   ctx_lens  device [B] int32: rows present per request, including the S query tokens'
 *             own rows (the last S).  Query j of request b sees rows t < L_b - S + 1 + j.
 *   topk_out  device [B][S][topk] int32: for each query the min(K, L) tokens with the
 *             largest score s(t) = sum_h w_h * max(0, q_h . k_t), ties to the lower token
 *             index, written in ascending token order and padded with -1.
 * The score formula is not printed on the pages; this is the reading the library takes.
 * Between calls the library keeps, per request slot and query, a guess of where the next
 * call's selection threshold lies (set from this call's scores or candidates).  A query with a
 * guess has its sweep list only the tokens scoring at or above it, and its select works from
 * that list alone when the list provably holds the answer (no segment overflowed and at
 * least K tokens listed); otherwise the query is rescored (a second sweep stores its scores)
 * and selected from all its scores.  The result is the same either way; the call launches
 * four kernels (two of which find nothing to do when every list serves), all on `stream`.
 * hs_hot_reset and hs_hot_release clear the guesses.
 */
hs_status hisparse_index_topk(hs_ctx* ctx, const void* q_idx, const float* w,
                              const int32_t* ctx_lens, int32_t B, int32_t S, int32_t* topk_out,
                              void* stream);

/*
 * Fused top-K resolver for B requests (one call per decode step; the S lists of a request
 * are resolved together, as MTP verification needs).  Per request, over the sorted union U
 * of its S top-K lists:
 *   - a token whose page is GPU-resident (block_table >= 0) gets row block*64 + offset and
 *     does not touch the LRU;
 *   - a token already in the hot buffer gets its slot's row, and the slot's LRU stamp is
 *     set to the request's step counter;
 *   - the remaining tokens (misses), in ascending token order, take the slots not touched
 *     in this call in least-recently-used order (empty slots first, ties to the lower slot);
 *     each copies its single row, for all n_layers layers, from the pinned host pool (host
 *     block from host_block_table) into that slot's row of the shared KV pool.  The copy is
 *     issued by the GPU; no CPU is involved.
 *   row_ids_out  device [B][S][topk] int32 rows into the shared KV pool, -1 where topk is -1
 *   stats_out    device [B][4] int32 (resident, hit, miss, hot pages in use) or NULL
 * The request's step counter then advances by one.  row_ids stays valid for
 * sparse_mla_decode until the next resolve of that request.
 */
hs_status hisparse_resolve(hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens, int32_t B,
                           int32_t S, int32_t* row_ids_out, int32_t* stats_out, void* stream);

/*
 * hisparse_resolve with plan windows (part-1 page, "Composing with the rest of vLLM":
 * speculative decoding runs on per-step resolver plans that can be replayed and share the
 * request's hot state).  A plan is the row_ids one call emits.  Reading taken: consecutive
 * calls of a request form a window; no slot touched by a call of the current window is given
 * to a miss, so every plan of the window stays valid (its rows keep their tokens and can be
 * gathered again, e.g. to replay sparse_mla_decode) until a call begins a new window, for
 * instance after drafts are rejected.
 *   begin_window  device [B] int32: nonzero where request b's call begins a new window; NULL
 *                 means every call begins one (hisparse_resolve)
 * The union of the selections of one window must fit the hot buffer; otherwise the misses
 * past the free slots are flagged HS_DEVERR_HOT_FULL and get row -1.
 */
hs_status hisparse_resolve_plan(hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens,
                                int32_t B, int32_t S, const int32_t* begin_window,
                                int32_t* row_ids_out, int32_t* stats_out, void* stream);

/*
 * Hot-buffer lifetime of single requests (part-1 page, "How it works": hot pages are taken
 * when a request first needs them and returned when it no longer does).
 *
 * hs_hot_release: for each of the n request slots in `reqs` (device [n] int32), in order,
 *   the request's hot buffer becomes cold, as after hs_hot_reset for that request alone:
 *   empty slots, LRU clock 0, no token mapped to a slot, a new plan window, no top-K guess.
 *   With hot_leasing its blocks go back to the end of the free-block pool in page order and
 *   its hot_blocks entries become -1.  A slot must be released before a new request reuses it;
 *   otherwise the old request's tokens would be found in its hot buffer.
 * hs_hot_pool_give: append the n blocks of `blocks` (device [n] int32; entries < 0 are
 *   skipped) to the end of the free-block pool, e.g. the blocks hisparse_release_pages freed
 *   or the blocks set aside for hot pages at start-up.  Blocks past the pool's capacity
 *   (num_gpu_blocks) are dropped with HS_DEVERR_POOL_FULL.
 * Leases happen inside hisparse_resolve / hisparse_resolve_plan: after the requests of a call
 * are resolved, the pages that got their first filled slot take blocks from the front of the
 * pool, request by request and page by page in ascending order.  An empty pool sets
 * HS_DEVERR_POOL_EMPTY and those rows read -1; the request should then be released.
 * Both calls allocate nothing and never synchronise; n = 0 is a no-op.  Host errors:
 * HS_ERR_INVALID_ARG (NULL ctx, n < 0, NULL list with n > 0), HS_ERR_STATE (not bound;
 * hs_hot_pool_give without hot_leasing).
 */
hs_status hs_hot_release(hs_ctx* ctx, const int32_t* reqs, int32_t n, void* stream);
hs_status hs_hot_pool_give(hs_ctx* ctx, const int32_t* blocks, int32_t n, void* stream);

/* Synchronise the context's device and copy the free-block pool, front first, into `out`
 * (host, room for `cap` entries); *n gets the number of free blocks (which may exceed cap).
 * For tests and inspection; never on the hot path.  HS_ERR_STATE without hot_leasing. */
hs_status hs_hot_pool_read(hs_ctx* ctx, int32_t* out, int32_t cap, int32_t* n);

/*
 * Sparse MLA decode attention of layer `layer` for B x S queries:
 *   out[b][j][h] = sum_k softmax_k(sm_scale * q[b][j][h] . latent(row_k)) * latent(row_k)[0:512]
 * over the rows row_ids[b][j][0 .. min(K, L_bj)).
 *   q        device [B][S][64][576] bf16
 *   row_ids  device [B][S][topk] int32 (from hisparse_resolve)
 *   ctx_lens device [B] int32 (as above)
 *   out      device [B][S][64][512] bf16
 *   lse      device [B][S][64] fp32 natural-log sum-exp of the scaled logits, or NULL
 */
hs_status sparse_mla_decode(hs_ctx* ctx, int32_t layer, const void* q, const int32_t* row_ids,
                            const int32_t* ctx_lens, int32_t B, int32_t S, float sm_scale,
                            void* out, float* lse, void* stream);

/*
 * Prefill of request slot b: the P new tokens that end its L-token context (rows and indexer
 * keys of all L tokens already written; every page resident).  Token i of the P (0-based) is
 * query i; it sees the rows t < L - P + 1 + i, causally, as a decode query sees its context.
 *
 * hisparse_prefill_index_topk: the indexer of every new token over every earlier token, the
 *   cost that grows with the square of the prompt (GLM-5.3 part-2 page, "PCP: split tokens,
 *   not heads", the paragraph on the indexer's cost), and the top-K of each, as
 *   hisparse_index_topk computes them for a decode query.
 *     q_idx     device [P][32][128] bf16;  w  device [P][32] fp32
 *     topk_out  device [P][topk] int32, ascending tokens, -1 padded
 * sparse_mla_prefill: sparse MLA attention of layer `layer` for the P tokens on the decode's
 *   MQA kernel: every row read serves all 64 heads (part-2 page, "Try it": with
 *   sparse_mla_force_mqa, prompts within the top-K stay on the sparse-MLA MQA kernel instead
 *   of dense MHA).
 *     q         device [P][64][576] bf16
 *     topk      device [P][topk] int32 (from hisparse_prefill_index_topk), or NULL for every
 *               row each token sees, which needs L <= topk (the prompt lies within top-K)
 *     out, lse  device [P][64][512] bf16 and [P][64] fp32 (lse may be NULL)
 * Both run the prompt in chunks of max_batch x max_queries tokens as decode-shaped groups of
 * max_queries tokens and use the context's top-K and decode scratch: do not overlap them with
 * step calls of the same context on other streams.  The request's hot state and top-K guesses
 * are untouched.  A placeholder page flags HS_DEVERR_BAD_BLOCK, a token a query cannot see
 * HS_DEVERR_BAD_ROW.  Host errors: HS_ERR_INVALID_ARG (b outside [0, max_batch), P < 1,
 * L < P, L past the block table, a NULL pointer, NULL topk with L > topk).
 */
hs_status hisparse_prefill_index_topk(hs_ctx* ctx, int32_t b, const void* q_idx, const float* w,
                                      int32_t L, int32_t P, int32_t* topk_out, void* stream);
hs_status sparse_mla_prefill(hs_ctx* ctx, int32_t layer, int32_t b, const void* q,
                             const int32_t* topk, int32_t L, int32_t P, float sm_scale, void* out,
                             float* lse, void* stream);

/*
 * sparse_mla_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same arguments, kernels
 * and results as sparse_mla_decode (bit for bit); its split-K partials live in a fixed scratch
 * array compiled into the library, 512 (query, split) partials (about 64 MiB) per device, held
 * by every device the library runs on until the process ends, instead of the bound workspace.
 * The split rule never needs more than the array holds (fewer than 256 queries use at most
 * 255 + queries partials; 256 queries or more use none); a call that would is refused with
 * HS_ERR_INVALID_ARG.  Every call on one device shares that device's array: calls that overlap
 * on one device (e.g. on two streams) race and must be ordered by the caller.  Allocates
 * nothing, never synchronises; the array's address is taken once per device at hs_create.
 */
hs_status sparse_mla_decode_noalloc(hs_ctx* ctx, int32_t layer, const void* q,
                                    const int32_t* row_ids, const int32_t* ctx_lens, int32_t B,
                                    int32_t S, float sm_scale, void* out, float* lse, void* stream);

/* Synchronise the context's device and read (then clear) the device error word. */
hs_status hs_read_device_error(hs_ctx* ctx, int32_t* code);

/* Device addresses of the hot-buffer state inside the bound workspace, for inspection (the
 * LRU state is part of what a resolve call produces).  Read-only for callers. */
typedef struct hs_hot_state_ptrs {
  const int32_t* slot_token;  /* [max_batch][hot_rows] token in each hot slot, -1 empty */
  const int32_t* slot_stamp;  /* [max_batch][hot_rows] LRU stamp, -1 never used */
  const int32_t* tok2slot;    /* [max_batch][tokens_per_req] hot slot of each token, -1 absent */
  const int32_t* req_step;    /* [max_batch] resolve calls made */
  int32_t hot_rows;
  int32_t reserved;
  int64_t tokens_per_req;     /* max_pages_per_req * 64 */
} hs_hot_state_ptrs;

hs_status hs_hot_state(const hs_ctx* ctx, hs_hot_state_ptrs* out);

/*
 * Write side of the host pool (part-1 page, "How it works", the paragraphs after the three
 * residency states: a completed cacheable prefix page is copied to host memory while the GPU
 * keeps serving it, all sparse-MLA layers in one launch after the forward pass, ordered on the
 * model's stream; under pressure the page later gives up its GPU block without a second copy).
 *
 * hisparse_materialize_pages: for each of the n entries (request b, page p) of `pages`
 *   (device [n][2] int32), copy the page's 64 rows of every layer from its GPU block
 *   (block_table[b][p]) into its host block (host_block_table[b][p], which the caller assigns
 *   beforehand).  The copy is issued by the GPU on `stream`; the pinned pool holds the rows once
 *   the stream has reached the end of the call.  An entry with no GPU block or no host block
 *   sets a device error bit and is skipped.
 * hisparse_release_pages: for each entry, if the page has a host block, set
 *   block_table[b][p] = -1 (the page becomes host-only: later selections of its tokens resolve
 *   through the hot buffer, copying from the host copy) and write the GPU block it held to
 *   freed_out[i] (device [n] int32); -1 where nothing was given up (already host-only, or a
 *   page listed twice).  The tail page, the one holding token ctx_lens[b] - 1, and pages past
 *   it are refused (HS_DEVERR_TAIL_PAGE), as is a resident page with no host block
 *   (HS_DEVERR_NO_HOST_COPY).  Materialise before releasing, on the same stream.
 * Both calls allocate nothing and never synchronise (graph-capturable like the step calls).
 * n = 0 is a no-op.  Host errors: HS_ERR_INVALID_ARG (NULL ctx, n < 0, NULL pages with n > 0,
 * NULL ctx_lens or freed_out), HS_ERR_STATE (context not bound, or no host pool).
 */
hs_status hisparse_materialize_pages(hs_ctx* ctx, const int32_t* pages, int32_t n, void* stream);
hs_status hisparse_release_pages(hs_ctx* ctx, const int32_t* pages, int32_t n,
                                 const int32_t* ctx_lens, int32_t* freed_out, void* stream);

/* Synchronise the context's device and read how many (request, query) selections of
 * hisparse_index_topk were made from the sweep's candidate list and how many from all the
 * scores, since the last hs_hot_reset (selections of L <= K or of invalid contexts are not
 * counted).  For measurement and tests; never on the hot path. */
hs_status hs_select_paths(hs_ctx* ctx, int64_t* from_candidates, int64_t* from_scores);

/* Number of split-K partitions sparse_mla_decode uses for a (B, S) batch. */
hs_status hs_decode_splits(const hs_ctx* ctx, int32_t B, int32_t S, int32_t* splits);

/* Per-kernel device timing, for measurement.  While enabled, every kernel launched by the
 * step calls (and hs_hot_reset) is bracketed by a pair of HIP events recorded on the caller's
 * stream, so the pair times that launch alone.  hs_kernel_times waits for the recorded events,
 * writes the summed milliseconds and the launch count of each kernel (indexed by
 * hs_kernel_id; `n` entries at most) since timing was enabled or last read, and starts a new
 * period.  Enabling creates a fixed pool of 16,384 events (no device memory); launches past
 * its capacity are not timed and hs_kernel_times then returns HS_ERR_STATE (counts written).
 * Disabling destroys the pool and drops unread records.  Off by default. */
typedef enum {
  HS_KERNEL_INDEX_SCORE = 0,  /* indexer sweep listing candidates above the guesses */
  HS_KERNEL_TOPK_SELECT = 1,  /* top-K select from the candidate lists */
  HS_KERNEL_RESOLVE = 2,      /* resolver: residency, hot hits, LRU victims, row ids */
  HS_KERNEL_MISS_COPY = 3,    /* host-to-device copy of the misses' rows */
  HS_KERNEL_DECODE = 4,       /* sparse MLA decode attention */
  HS_KERNEL_DECODE_MERGE = 5, /* split-K merge of the decode */
  HS_KERNEL_HOT_RESET = 6,    /* hot-buffer reset */
  HS_KERNEL_MATERIALIZE = 7,  /* device-to-host copy of completed pages */
  HS_KERNEL_RELEASE = 8,      /* pages giving up their GPU blocks */
  HS_KERNEL_LEASE = 9,        /* hot pages taking blocks from the free-block pool */
  HS_KERNEL_HOT_RELEASE = 10, /* requests' hot buffers made cold, blocks returned */
  HS_KERNEL_POOL_GIVE = 11,   /* blocks appended to the free-block pool */
  HS_KERNEL_INDEX_RESCORE = 12, /* indexer sweep storing scores (queries the lists cannot serve) */
  HS_KERNEL_TOPK_RESCORED = 13, /* top-K select of those queries from their scores */
  HS_KERNEL_COUNT = 14
} hs_kernel_id;

hs_status hs_kernel_timing(hs_ctx* ctx, int32_t enable);
hs_status hs_kernel_times(hs_ctx* ctx, double* ms, int64_t* launches, int32_t n);

/* Measurement helper, not part of the decode step: the best of `reps` streaming reads of the
 * device buffer `buf` (`bytes`, 16-byte aligned; each 16-byte piece read once per pass) on the
 * current device's null stream, in GB/s.  `sink` is a device word the reads are folded into
 * (written only in the unlikely case the fold meets a fixed constant).  Synchronises. */
hs_status hs_measure_read_gbps(const void* buf, size_t bytes, void* sink, int32_t reps, double* gbps);

const char* hs_status_string(hs_status status);
const char* hs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
