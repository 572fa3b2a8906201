// Write side of the pinned host pool (gfx950).
//
// What is computed (Hybrid HiSparse part-1 page, "How it works", the two paragraphs after the
// three residency states): when a cacheable prefix page completes, its rows are copied to host
// memory while the GPU keeps serving the page, every sparse-MLA layer of the listed pages in
// one launch after the forward pass, ordered on the model's stream.  If the GPU pool fills
// later, the page gives up its GPU block without a second copy: its block-table entry becomes
// a placeholder, and from then on its tokens are read from the host copy through the hot
// buffer.  The tail page (the one holding the newest token) is never given up ("Three KV
// residency states": the tail is never evicted).
//
// Materialisation: every (page, layer) block of the list is copied by the GPU, 16 bytes per
// work item over the whole grid, eight loads in flight per thread, from HBM into the mapped
// host pool (PCIe writes).  Release: one thread per entry swaps the block-table entry for the
// placeholder and reports the block it held.
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kMatThreads = 256;
constexpr int kMatBlocks = 256;

__global__ __launch_bounds__(kMatThreads) void materialize_kernel(
    const int32_t* __restrict__ pages, int n, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ host_block_table, int max_batch, int max_pages,
    const uint8_t* __restrict__ kv_pool, uint8_t* __restrict__ host_pool, int n_layers, int row_bytes,
    int64_t num_gpu_blocks, int64_t num_host_blocks, int32_t* __restrict__ err) {
  const int pieces = kBlock * row_bytes / 16;  // 16-byte pieces of one block of one layer
  const int64_t per_entry = (int64_t)n_layers * pieces;
  const int64_t total = (int64_t)n * per_entry;
  const int64_t gpu_layer = num_gpu_blocks * kBlock * (int64_t)row_bytes;
  const int64_t host_layer = num_host_blocks * kBlock * (int64_t)row_bytes;
  const int64_t stride = (int64_t)gridDim.x * kMatThreads;
  constexpr int kBatch = 8;
  for (int64_t base = (int64_t)blockIdx.x * kMatThreads + threadIdx.x; base < total; base += stride * kBatch) {
    u32x4 v[kBatch];
    int64_t dst[kBatch];
#pragma unroll
    for (int e = 0; e < kBatch; ++e) {
      const int64_t idx = base + e * stride;
      dst[e] = -1;
      if (idx < total) {
        const int i = (int)(idx / per_entry);
        const int rem = (int)(idx - (int64_t)i * per_entry);
        const int layer = rem / pieces, q = rem - layer * pieces;
        const int b = pages[2 * i], p = pages[2 * i + 1];
        int32_t g = -1, h = -1;
        if (b >= 0 && b < max_batch && p >= 0 && p < max_pages) {
          g = block_table[(int64_t)b * max_pages + p];
          h = host_block_table[(int64_t)b * max_pages + p];
        }
        const bool ok = g >= 0 && g < num_gpu_blocks && h >= 0 && h < num_host_blocks;
        if (!ok && rem == 0) raise_error(err, g < 0 || g >= num_gpu_blocks ? HS_DEVERR_BAD_BLOCK : HS_DEVERR_NO_HOST_COPY);
        if (ok) {
          v[e] = *reinterpret_cast<const u32x4*>(kv_pool + layer * gpu_layer + (int64_t)g * kBlock * row_bytes + q * 16);
          dst[e] = layer * host_layer + (int64_t)h * kBlock * row_bytes + q * 16;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kBatch; ++e)
      if (dst[e] >= 0) __builtin_nontemporal_store(v[e], reinterpret_cast<u32x4*>(host_pool + dst[e]));
  }
}

__global__ __launch_bounds__(256) void release_kernel(
    const int32_t* __restrict__ pages, int n, const int32_t* __restrict__ ctx_lens,
    int32_t* __restrict__ block_table, const int32_t* __restrict__ host_block_table, int max_batch,
    int max_pages, int64_t num_host_blocks, int32_t* __restrict__ freed, int32_t* __restrict__ err) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int b = pages[2 * i], p = pages[2 * i + 1];
  int32_t out = -1;
  if (b < 0 || b >= max_batch || p < 0 || p >= max_pages) {
    raise_error(err, HS_DEVERR_BAD_BLOCK);
  } else if (p >= (ctx_lens[b] - 1) / kBlock) {
    raise_error(err, HS_DEVERR_TAIL_PAGE);  // the tail page, or a page past the context
  } else {
    const int64_t k = (int64_t)b * max_pages + p;
    const int32_t h = host_block_table[k];
    if (h < 0 || h >= num_host_blocks) {
      if (block_table[k] >= 0) raise_error(err, HS_DEVERR_NO_HOST_COPY);
    } else {
      // exchange, so that a page listed twice is given up once
      out = atomicExch(&block_table[k], -1);
      if (out < 0) out = -1;
    }
  }
  freed[i] = out;
}

}  // namespace
}  // namespace hs

using namespace hs;

hipError_t hs_launch_materialize(const hs_ctx* ctx, const int32_t* pages, int n, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  hs_timer_mark(ctx, HS_KERNEL_MATERIALIZE, true, stream);
  hipLaunchKernelGGL(materialize_kernel, dim3(kMatBlocks), dim3(kMatThreads), 0, stream, pages, n,
                     ctx->buf.block_table, ctx->buf.host_block_table, c.max_batch, c.max_pages_per_req,
                     static_cast<const uint8_t*>(ctx->buf.kv_pool), static_cast<uint8_t*>(ctx->host_pool_dev),
                     c.n_layers, ctx->row_bytes, (int64_t)c.num_gpu_blocks, (int64_t)c.num_host_blocks,
                     ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_MATERIALIZE, false, stream);
  return hipGetLastError();
}

hipError_t hs_launch_release(const hs_ctx* ctx, const int32_t* pages, int n, const int32_t* ctx_lens,
                             int32_t* freed, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  hs_timer_mark(ctx, HS_KERNEL_RELEASE, true, stream);
  hipLaunchKernelGGL(release_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pages, n,
                     ctx_lens, ctx->buf.block_table, ctx->buf.host_block_table, c.max_batch,
                     c.max_pages_per_req, (int64_t)c.num_host_blocks, freed, ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_RELEASE, false, stream);
  return hipGetLastError();
}
