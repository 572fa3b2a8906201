// Sparse MLA decode attention over resolved rows (gfx950).
//
// What is computed (GLM-5.3 part-2 page, "Why not TP or DP?": MLA's latent row is shared by
// all 64 heads; "Try it": the sparse-MLA kernel in MQA form; footnote 1: QK over 576 dims, PV
// over 512): for each query token and head h,
//     out_h = sum_k softmax_k(sm_scale * q_h . x_k) * x_k[0:512]
// over the selected latent rows x_k, with the row ids emitted by the resolver.
//
// FP8 rows (656 bytes) hold 512 E4M3 codes c with one fp32 scale a, and 64 bf16 rope values.
// The per-row scale is folded out of the contractions: q . x = a (q_nope . c) + q_rope . rope,
// and sum_k p_k x_k = sum_k (p_k a_k) c_k, so the MFMAs see exactly converted bf16 codes.
//
// Workgroup = (query token, split of its rows), 4 waves; wave w owns heads 16w .. 16w+15 and
// keeps its 16 x 576 query slice in registers.  Rows are processed in tiles of 64: the tile is
// gathered from HBM once (8-byte pieces of 8 rows per thread, coalesced along the row) and
// written to LDS twice, row-major for QK and transposed (dim-major) for PV, the transpose done
// in registers with byte permutes.  Each wave computes S^T = K Q^T and O^T = V^T P^T on 16x16x32
// bf16 MFMAs; in that orientation a lane owns one head, so the online-softmax state is
// per-lane and the probabilities feed the PV MFMA straight from registers (the PV k-slots
// are assigned to rows in the order the QK result lays them out, and the transposed V tile
// is stored in the same order).  Splits of one query are combined with log-sum-exp, the same
// algebra as merging per-shard partial attention (part-2 page, "DCP" section).
#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kDecThreads = 256;

template <bool kFp8>
struct DecodeLds {
  static constexpr int kNopeStride = kFp8 ? 528 : 1040;  // bytes per row of the nope part
  static constexpr int kRopeStride = 144;                 // 64 bf16 + pad
  static constexpr int kVtStride = kFp8 ? 72 : 144;       // bytes per dim of the transposed tile
  static constexpr int kNopeBytes = kTileRows * kNopeStride;
  static constexpr int kRopeBytes = kTileRows * kRopeStride;
  static constexpr int kVtBytes = kDv * kVtStride;
  static constexpr int kOffRope = kNopeBytes;
  static constexpr int kOffVt = kOffRope + kRopeBytes;
  static constexpr int kOffScale = kOffVt + kVtBytes;
  static constexpr int kOffRid = kOffScale + kTileRows * 4;
  static constexpr int kTotal = kOffRid + kTileRows * 4;
};

// Gather one 64-row tile into LDS (both layouts).  Rows at positions >= n_tile are zero.
template <bool kFp8>
__device__ __forceinline__ void gather_tile(const uint8_t* __restrict__ kv, unsigned char* lds,
                                            const int32_t* __restrict__ rid_src, int n_tile,
                                            int64_t n_rows_pool, int32_t* err) {
  using Lds = DecodeLds<kFp8>;
  constexpr int kRow = kFp8 ? kFp8Row : kBf16Row;
  const int tid = threadIdx.x;
  int32_t* rid = reinterpret_cast<int32_t*>(lds + Lds::kOffRid);
  float* scale = reinterpret_cast<float*>(lds + Lds::kOffScale);
  if (tid < kTileRows) {
    int32_t r = tid < n_tile ? rid_src[tid] : -1;
    if (r >= n_rows_pool || (tid < n_tile && r < 0)) {
      raise_error(err, HS_DEVERR_BAD_ROW);
      r = -1;
    }
    rid[tid] = r;
    float a = 0.0f;
    if (kFp8 && r >= 0) a = *reinterpret_cast<const float*>(kv + (int64_t)r * kRow + 640);
    scale[tid] = a;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int e = tid + kDecThreads * it;
    const int dg = e & 63, rg = e >> 6;
    const int kap = rg >> 2, g = rg & 3;
    int rows[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rows[i] = 32 * kap + 4 * g + i;
      rows[4 + i] = 32 * kap + 16 + 4 * g + i;
    }
    if constexpr (kFp8) {
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t r = rid[rows[i]];
        u32x2 v = {0u, 0u};
        if (r >= 0) v = *reinterpret_cast<const u32x2*>(kv + (int64_t)r * kRow + 8 * dg);
        lo[i] = v[0];
        hi[i] = v[1];
        *reinterpret_cast<u32x2*>(lds + rows[i] * Lds::kNopeStride + 8 * dg) = v;
      }
      uint32_t a[4], bq[4], c[4], d[4];
      transpose4x4_bytes(lo[0], lo[1], lo[2], lo[3], a[0], a[1], a[2], a[3]);
      transpose4x4_bytes(lo[4], lo[5], lo[6], lo[7], bq[0], bq[1], bq[2], bq[3]);
      transpose4x4_bytes(hi[0], hi[1], hi[2], hi[3], c[0], c[1], c[2], c[3]);
      transpose4x4_bytes(hi[4], hi[5], hi[6], hi[7], d[0], d[1], d[2], d[3]);
      unsigned char* vt = lds + Lds::kOffVt + 32 * kap + 8 * g;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        *reinterpret_cast<u32x2*>(vt + (8 * dg + k) * Lds::kVtStride) = u32x2{a[k], bq[k]};
        *reinterpret_cast<u32x2*>(vt + (8 * dg + 4 + k) * Lds::kVtStride) = u32x2{c[k], d[k]};
      }
    } else {
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t r = rid[rows[i]];
        v[i] = u32x4{0u, 0u, 0u, 0u};
        if (r >= 0) v[i] = *reinterpret_cast<const u32x4*>(kv + (int64_t)r * kRow + 16 * dg);
        *reinterpret_cast<u32x4*>(lds + rows[i] * Lds::kNopeStride + 16 * dg) = v[i];
      }
      unsigned char* vt = lds + Lds::kOffVt + 2 * (32 * kap + 8 * g);
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        u32x4 even, odd;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          uint32_t c0, c1;
          transpose2x2_u16(v[2 * pr][dw], v[2 * pr + 1][dw], c0, c1);
          even[pr] = c0;
          odd[pr] = c1;
        }
        *reinterpret_cast<u32x4*>(vt + (8 * dg + 2 * dw) * Lds::kVtStride) = even;
        *reinterpret_cast<u32x4*>(vt + (8 * dg + 2 * dw + 1) * Lds::kVtStride) = odd;
      }
    }
  }
  // rope: 64 rows x 128 bytes (bf16) in 16-byte pieces
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int cidx = tid + kDecThreads * it;
    const int row = cidx >> 3, part = cidx & 7;
    const int32_t r = rid[row];
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r >= 0) v = *reinterpret_cast<const u32x4*>(kv + (int64_t)r * kRow + (kFp8 ? 512 : 1024) + 16 * part);
    *reinterpret_cast<u32x4*>(lds + Lds::kOffRope + row * Lds::kRopeStride + 16 * part) = v;
  }
  __syncthreads();
}

template <bool kFp8>
__global__ __launch_bounds__(kDecThreads) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ row_ids,
    const int32_t* __restrict__ ctx_lens, int S, int K, int max_ctx,
    const uint8_t* __restrict__ kv, int64_t n_rows_pool, float qk_scale_log2, int splits,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int32_t* __restrict__ err) {
  using Lds = DecodeLds<kFp8>;
  extern __shared__ __align__(16) unsigned char lds[];

  const int bj = blockIdx.x / splits, sp = blockIdx.x % splits;
  const int b = bj / S, j = bj % S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int head = 16 * wave + col;

  const int Lb = ctx_lens[b];
  int n = 0;
  if (Lb >= S && Lb <= max_ctx) n = min(K, Lb - S + 1 + j);
  else if (tid == 0 && sp == 0) raise_error(err, HS_DEVERR_SHORT_CONTEXT);
  const int per = ((n + splits - 1) / splits + kTileRows - 1) / kTileRows * kTileRows;
  const int r0 = sp * per, r1 = min(n, r0 + per);

  // Q^T fragments: B operand, k-slots 8g..8g+7 of k-step s = dims 32s + 8g .. +8.
  bf16x8 qf[18];
  const uint16_t* qp = q + ((int64_t)bj * kHeads + head) * kDqk + 8 * g;
#pragma unroll
  for (int s = 0; s < 18; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 32 * s));

  f32x4 o[32];
#pragma unroll
  for (int m = 0; m < 32; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.0f;

  const int32_t* rids = row_ids + (int64_t)bj * K;
  const float* scale = reinterpret_cast<const float*>(lds + Lds::kOffScale);
  for (int t0 = r0; t0 < r1; t0 += kTileRows) {
    const int n_tile = min(kTileRows, r1 - t0);
    gather_tile<kFp8>(kv, lds, rids + t0, n_tile, n_rows_pool, err);

    // ---- S^T = K Q^T for the 64 rows; lane holds rows 16 sig + 4 g + i of head `col`
    float s2[4][4];
#pragma unroll
    for (int sig = 0; sig < 4; ++sig) {
      const int ra = 16 * sig + col;
      f32x4 c1 = {0.f, 0.f, 0.f, 0.f}, c2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        bf16x8 a;
        if constexpr (kFp8) {
          const u32x2 kb = *reinterpret_cast<const u32x2*>(lds + ra * Lds::kNopeStride + 32 * s + 8 * g);
          a = e4m3x8_to_bf16(kb[0], kb[1]);
        } else {
          a = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + ra * Lds::kNopeStride + 64 * s + 16 * g));
        }
        c1 = mfma16x16x32(a, qf[s], c1);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            lds + Lds::kOffRope + ra * Lds::kRopeStride + 64 * s + 16 * g));
        c2 = mfma16x16x32(a, qf[16 + s], c2);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * sig + 4 * g + i;
        const float a = kFp8 ? scale[r] : 1.0f;
        s2[sig][i] = r < n_tile ? (a * c1[i] + c2[i]) * qk_scale_log2 : -INFINITY;
      }
    }
    // ---- online softmax (per head = per lane column; rows spread over the 4 lane groups)
    float tmax = s2[0][0];
#pragma unroll
    for (int sig = 0; sig < 4; ++sig)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s2[sig][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_part *= alpha;
#pragma unroll
    for (int m = 0; m < 32; ++m) o[m] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int sig = 0; sig < 4; ++sig)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s2[sig][i] - m_new);
        l_part += p;
        const float a = kFp8 ? scale[16 * sig + 4 * g + i] : 1.0f;
        pb[sig >> 1][(sig & 1) * 4 + i] = (__bf16)(p * a);
      }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        bf16x8 a;
        const unsigned char* vp = lds + Lds::kOffVt + (16 * m + col) * Lds::kVtStride;
        if constexpr (kFp8) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(vp + 32 * kap + 8 * g);
          a = e4m3x8_to_bf16(v[0], v[1]);
        } else {
          a = as_bf16x8(*reinterpret_cast<const u32x4*>(vp + 2 * (32 * kap + 8 * g)));
        }
        o[m] = mfma16x16x32(a, pb[kap], o[m]);
      }
    }
    __syncthreads();  // the tile's LDS is reused by the next gather
  }

  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (splits == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* op = out + ((int64_t)bj * kHeads + head) * kDv;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const __bf16 v0 = (__bf16)(o[m][0] * inv), v1 = (__bf16)(o[m][1] * inv);
      const __bf16 v2 = (__bf16)(o[m][2] * inv), v3 = (__bf16)(o[m][3] * inv);
      const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
      const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
      *reinterpret_cast<u32x2*>(op + 16 * m + 4 * g) = u32x2{w0, w1};
    }
    if (lse && g == 0) lse[(int64_t)bj * kHeads + head] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
  } else {
    const int64_t part = (int64_t)bj * splits + sp;
    if (g == 0) {
      part_ml[(part * kHeads + head) * 2 + 0] = m_run;
      part_ml[(part * kHeads + head) * 2 + 1] = l_tot;
    }
    if (r1 > r0) {
      float* pp = part_o + (part * kHeads + head) * kDv;
#pragma unroll
      for (int m = 0; m < 32; ++m) *reinterpret_cast<f32x4*>(pp + 16 * m + 4 * g) = o[m];
    }
  }
}

// Combine the split partials of each query: M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           int splits, uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int bj = blockIdx.x;
  const int h = threadIdx.x >> 2, qtr = threadIdx.x & 3;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    const float* ml = part_ml + (((int64_t)bj * splits + s) * kHeads + h) * 2;
    if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
  }
  float L = 0.0f;
  float f[kMaxSplits];
  for (int s = 0; s < splits; ++s) {
    const float* ml = part_ml + (((int64_t)bj * splits + s) * kHeads + h) * 2;
    f[s] = ml[1] > 0.0f ? exp2f(ml[0] - M) : 0.0f;
    L += ml[1] * f[s];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint16_t* op = out + ((int64_t)bj * kHeads + h) * kDv + 128 * qtr;
  for (int d = 0; d < 128; d += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
      if (f[s] == 0.0f) continue;
      const f32x4 v = *reinterpret_cast<const f32x4*>(
          part_o + (((int64_t)bj * splits + s) * kHeads + h) * kDv + 128 * qtr + d);
      acc += v * f[s];
    }
    uint32_t w0, w1;
    {
      const __bf16 v0 = (__bf16)(acc[0] * inv), v1 = (__bf16)(acc[1] * inv);
      const __bf16 v2 = (__bf16)(acc[2] * inv), v3 = (__bf16)(acc[3] * inv);
      w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
      w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
    }
    *reinterpret_cast<u32x2*>(op + d) = u32x2{w0, w1};
  }
  if (lse && qtr == 0) lse[(int64_t)bj * kHeads + h] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace
}  // namespace hs

using namespace hs;

size_t hs_decode_lds_bytes(int kv_dtype) {
  return kv_dtype == HS_FP8_E4M3 ? DecodeLds<true>::kTotal : DecodeLds<false>::kTotal;
}

int hs_choose_splits(const hs_ctx* ctx, int B, int S) {
  const int nq = B * S;
  const int tiles = (ctx->cfg.topk + kTileRows - 1) / kTileRows;
  int splits = (512 + nq - 1) / nq;
  if (splits > tiles) splits = tiles;
  if (splits > ctx->lay.splits_cap) splits = ctx->lay.splits_cap;
  if (splits < 1) splits = 1;
  return splits;
}

hipError_t hs_launch_decode(const hs_ctx* ctx, int layer, const void* q, const int32_t* row_ids,
                            const int32_t* ctx_lens, int B, int S, float sm_scale, void* out,
                            float* lse, int splits, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  const int64_t n_rows_pool = c.num_gpu_blocks * kBlock;
  const uint8_t* kv = static_cast<const uint8_t*>(ctx->buf.kv_pool) +
                      (int64_t)layer * n_rows_pool * ctx->row_bytes;
  const float qk_scale_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(B * S * splits)), block(kDecThreads);
  if (c.kv_dtype == HS_FP8_E4M3)
    hipLaunchKernelGGL(sparse_mla_decode_kernel<true>, grid, block, DecodeLds<true>::kTotal, stream,
                       static_cast<const uint16_t*>(q), row_ids, ctx_lens, S, c.topk,
                       c.max_pages_per_req * kBlock, kv, n_rows_pool, qk_scale_log2, splits,
                       static_cast<uint16_t*>(out), lse, ctx->ws.part_o, ctx->ws.part_ml,
                       ctx->ws.err);
  else
    hipLaunchKernelGGL(sparse_mla_decode_kernel<false>, grid, block, DecodeLds<false>::kTotal,
                       stream, static_cast<const uint16_t*>(q), row_ids, ctx_lens, S, c.topk,
                       c.max_pages_per_req * kBlock, kv, n_rows_pool, qk_scale_log2, splits,
                       static_cast<uint16_t*>(out), lse, ctx->ws.part_o, ctx->ws.part_ml,
                       ctx->ws.err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B * S)), dim3(256), 0, stream,
                     ctx->ws.part_o, ctx->ws.part_ml, splits, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

// Raise the dynamic-LDS limit of the kernels that need more than the default.
hipError_t hs_set_kernel_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_mla_decode_kernel<true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     DecodeLds<true>::kTotal);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_mla_decode_kernel<false>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, DecodeLds<false>::kTotal);
}
