// Internal declarations of the HiSparse decode-step library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hs {

// Fixed shapes of the kernels.
constexpr int kBlock = 64;             // tokens per page
constexpr int kIdxHeads = 32;          // indexer heads
constexpr int kIdxDim = 128;           // indexer head dim
constexpr int kHeads = 64;             // MLA query heads sharing one latent row
constexpr int kDqk = 576;              // latent: 512 "nope" + 64 rope
constexpr int kDv = 512;               // value = first 512 latent dims
constexpr int kFp8Row = 656;           // FP8 latent row bytes
constexpr int kBf16Row = 1152;         // bf16 latent row bytes
constexpr int kIdxFp8Block = 8448;     // 64 x 128 e4m3 + 64 fp32 scales
constexpr int kIdxBf16Block = 16384;   // 64 x 128 bf16
constexpr int kMaxTopk = 2048;
constexpr int kMaxQueries = 4;
constexpr int kMaxUnion = kMaxTopk * kMaxQueries;
constexpr int kMaxHot = 16384;

// Top-K radix select: the first digit is score bits [30:19] (8 exponent + 4 mantissa bits of
// a non-negative fp32), histogrammed by the score sweep itself.
constexpr int kHistBins = 4096;
constexpr int kHistShift = 19;
constexpr int kPagesPerItem = 64;      // pages scored by one sweep workgroup (4,096 tokens)
constexpr int kDefaultCandCap = 4096;  // on-chip candidates of the threshold bin
// Candidate list of the select: each sweep wave writes the tokens whose score key reaches the
// query's guess into its own segment (192 entries) of the query's list.
constexpr int kSegCap = 192;
constexpr int kSweepWaves = 4;
constexpr uint32_t kGuessOff = 0xFFFFFFFFu;  // no guess: no candidates are written

constexpr int kZeroRowBytes = 1024;  // >= one FP8 row (656 bytes)

// Decode split-K.
constexpr int kTileRows = 64;
constexpr int kMaxSplits = 32;
// sparse_mla_decode_noalloc: (query, split) partials the fixed scratch holds.  The split rule
// (hs_choose_splits) keeps queries x splits below 256 + queries for fewer than 256 queries and
// uses no partials from 256 queries on, so every call fits.
constexpr int kFixedPartials = 512;
constexpr int kMaxDevices = 64;

// Pointers into the borrowed device workspace.
struct Workspace {
  int32_t* slot_token;   // [Bmax][H]          token held by each hot slot, -1 empty
  int32_t* slot_stamp;   // [Bmax][H]          LRU stamp (resolve call counter), -1 never
  int32_t* lru_order;    // [2][Bmax][H]       slots in (stamp, slot) order, double-buffered by
                         //                    the parity of the request's call counter
  int32_t* tok2slot;     // [Bmax][Lmax]       hot slot of each token, -1 absent
  int32_t* req_step;     // [Bmax]             resolve calls made per request
  int32_t* req_used;     // [Bmax]             hot slots ever filled per request
  int32_t* win_start;    // [Bmax]             call counter at which the current plan window began
  int32_t* pool_ring;    // [num_gpu_blocks]   free-block pool (hot_leasing), a ring
  int64_t* pool_ctr;     // [2]                pool front and back, monotonic (entry = ring[x % cap])
  int32_t* err;          // [1]                sticky device error word (HS_DEVERR_*)
  float* scores;         // [Bmax][Smax][Lmax] indexer scores of one call
  uint32_t* bitmap;      // [Bmax][Smax][bm_words] selected-token bitmap
  int32_t* miss_src;     // [Bmax][Smax*K] host row of each miss of the last resolve
  int32_t* miss_dst;     // [Bmax][Smax*K] device row (hot slot) it is copied to
  int32_t* miss_cnt;     // [Bmax] misses of the last resolve
  float* part_o;         // [Bmax*Smax*splits_cap][64][512] split-K partial outputs
  float* part_ml;        // [Bmax*Smax*splits_cap][64][2] split-K (max, sum) in log2 units
  uint32_t* guess;       // [Bmax][Smax]       score key from which the sweep lists candidates
  int32_t* rescore;      // [Bmax][Smax]       queries the candidate lists could not serve this call
  int32_t* n_rescore;    // [1]                how many of them (follows `rescore`)
  uint32_t* seg_count;   // [Bmax][Smax][n_seg] candidates each sweep wave found (> kSegCap: overflow)
  uint64_t* cands;       // [Bmax][Smax][n_seg][kSegCap] (key << 32) | ~token
  unsigned long long* path_count;  // [2] selections made from the candidate list / the scores
  uint8_t* zero_row;     // [kZeroRowBytes]    zeros: what a skipped row of the decode reads
  // prefill, run as decode-shaped groups of max_queries queries
  int32_t* pf_lens;      // [Bmax]             context length of each group
  uint32_t* pf_guess;    // [Bmax][Smax]       the groups' top-K guesses (off)
  unsigned long long* pf_paths;  // [2]        selection paths of prefill calls
  int32_t* pf_rows;      // [Bmax][Smax][K]    row ids of a prefill chunk's selections
};

struct Layout {
  size_t off_slot_token, off_slot_stamp, off_lru_order, off_tok2slot, off_req_step, off_req_used,
      off_win_start, off_pool_ring, off_pool_ctr, off_err, off_scores, off_bitmap, off_miss_src, off_miss_dst, off_miss_cnt,
      off_part_o, off_part_ml, off_guess, off_rescore, off_seg_count, off_cands, off_path_count, off_zero_row,
      off_pf_lens, off_pf_guess, off_pf_paths, off_pf_rows, total;
  int32_t hot_rows;
  int64_t lmax;       // max_pages_per_req * 64
  int64_t bm_words;   // bitmap words per (request, query): lmax rounded up to 1,024, / 32
  int32_t splits_cap;
  int32_t n_seg;      // candidate segments per (request, query): sweep workgroups x waves
};

hs_status compute_layout(const hs_config& c, Layout* out);

}  // namespace hs

namespace hs {
struct KernelTimer;  // per-kernel event timing (hs_api.cpp)
}  // namespace hs

struct hs_ctx {
  hs_config cfg;
  hs::Layout lay;
  int device;
  int row_bytes;
  int idx_block_bytes;
  void* host_pool;          // host address (pinned, mapped)
  void* host_pool_dev;      // device address of the same memory
  size_t host_pool_bytes;
  bool bound;
  hs_buffers buf;
  hs::Workspace ws;
  hs::KernelTimer* timer;   // null unless hs_kernel_timing enabled it
};

// Brackets one kernel launch with timing events when the context's timer is enabled
// (begin = true before the launch, false after it); a no-op otherwise.
void hs_timer_mark(const hs_ctx* ctx, int kernel, bool begin, hipStream_t stream);

// Kernel launchers (each enqueues on `stream`, returns hipSuccess or the launch error).
hipError_t hs_launch_hot_reset(const hs_ctx* ctx, hipStream_t stream);
hipError_t hs_launch_index_topk(const hs_ctx* ctx, const void* q_idx, const float* w,
                                const int32_t* ctx_lens, int B, int S, int32_t* topk_out,
                                hipStream_t stream);
hipError_t hs_launch_resolve(const hs_ctx* ctx, const int32_t* topk, const int32_t* ctx_lens, int B,
                             int S, const int32_t* begin_window, int32_t* row_ids, int32_t* stats,
                             hipStream_t stream);
hipError_t hs_launch_hot_release(const hs_ctx* ctx, const int32_t* reqs, int n, hipStream_t stream);
hipError_t hs_launch_pool_give(const hs_ctx* ctx, const int32_t* blocks, int n, hipStream_t stream);
hipError_t hs_launch_decode(const hs_ctx* ctx, int layer, const void* q, const int32_t* row_ids,
                            const int32_t* ctx_lens, int B, int S, float sm_scale, void* out,
                            float* lse, int splits, hipStream_t stream, float* part_o = nullptr,
                            float* part_ml = nullptr);
// The fixed scratch of sparse_mla_decode_noalloc: its device address on `device`, taken once
// with that device current (hs_create does it); nullptr before that.
hipError_t hs_fixed_scratch_init(int device);
void* hs_fixed_scratch(int device);
int hs_choose_splits(const hs_ctx* ctx, int B, int S);
hipError_t hs_launch_materialize(const hs_ctx* ctx, const int32_t* pages, int n, hipStream_t stream);
hipError_t hs_launch_release(const hs_ctx* ctx, const int32_t* pages, int n, const int32_t* ctx_lens,
                             int32_t* freed, hipStream_t stream);
int hs_select_cand_cap(const hs_config& c);
hipError_t hs_launch_prefill_lens(const hs_ctx* ctx, int L, int P, int c0, int n, hipStream_t stream);
hipError_t hs_launch_prefill_index_topk(const hs_ctx* ctx, int b, const void* q_idx, const float* w,
                                        int L, int P, int32_t* topk_out, hipStream_t stream);
hipError_t hs_launch_prefill_decode(const hs_ctx* ctx, int layer, int b, const void* q,
                                    const int32_t* topk, int L, int P, float sm_scale, void* out,
                                    float* lse, hipStream_t stream);
