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
// and sum_k p_k x_k = sum_k (p_k a_k) c_k, so the MFMAs see the codes converted exactly.
//
// Both kernels: workgroup = (query token, split of its rows); rows go in tiles of 64; in the
// MFMA orientation S^T = K Q^T and O^T += V^T P^T a lane owns one head, so the softmax state is
// per lane and the probabilities feed the PV MFMA in the layout the QK result has (the PV
// k-slots are assigned to rows in that order).  The running maximum is only moved when it grows
// by more than 2^8, so the accumulators are rarely rescaled.  Splits of one query are combined
// with log-sum-exp, the same algebra as merging per-shard partial attention (part-2 page, "DCP"
// section).
//
// FP8 rows (sparse_mla_decode_fp8_kernel, below): 8 waves, 4 that score (QK and the softmax, 16
// heads each) and 4 that accumulate (PV, 128 value dims each), working on consecutive tiles;
// tiles stay FP8 in LDS, in a ring of three filled by direct loads one tile ahead.
//
// bf16 rows (sparse_mla_decode_kernel): 4 waves = 2 head groups (32 heads each) x 2 halves.  A
// tile is gathered from HBM once (8-byte pieces of 8 rows per thread, coalesced along the row)
// and written to LDS twice: row-major for QK and dim-major for PV (transposed in registers).
// Each wave computes S^T for its 32 heads on half the tile's rows and O^T for its 32 heads on
// half the value dims over all the rows, on 32x32x16 bf16 MFMAs; the two waves of a head group
// swap their row maxima and probabilities through LDS.
#include <mutex>

#include "hs_device.h"
#include "hs_internal.h"

namespace hs {
namespace {

constexpr int kDecThreads = 256;
constexpr float kLazyRescale = 8.0f;  // log2 units

// LDS of one tile (bf16 after conversion).
struct DecLds {
  static constexpr int kKStride = kDqk * 2 + 16;          // bytes per row: 576 bf16 + pad
  static constexpr int kVtStride = kTileRows * 2 + 16;    // bytes per dim: 64 bf16 + pad
  static constexpr int kOffVt = kTileRows * kKStride;
  static constexpr int kOffScale = kOffVt + kDv * kVtStride;
  static constexpr int kOffRid = kOffScale + kTileRows * 4;
  static constexpr int kTotal = kOffRid + kTileRows * 4;
};
static_assert(DecLds::kTotal <= 160 * 1024, "decode LDS");

// Position in the transposed tile of row r (0..63): within each 32-row half, 16-row k-steps;
// within a k-step, lane half hf holds rows {4hf..4hf+3, 8+4hf..8+4hf+3} at 8 hf .. 8 hf + 7.
__device__ __forceinline__ int vt_pos(int r) {
  const int rh = r >> 5, kap = (r >> 4) & 1, q = r & 15;
  const int hf = (q >> 2) & 1, e = (q & 3) + ((q >> 3) << 2);
  return 32 * rh + 16 * kap + 8 * hf + e;
}

// Thread work of a gather: two blocks of 8 rows x 8 dims (nope part) and two 16-byte rope
// pieces.  Block g = tid + 256 it: dim group dg = g % 64, row group rg = g / 64 whose 8 rows are
// the ones stored at transposed positions 8 rg .. 8 rg + 7.
template <bool kFp8>
struct TileRegs {
  u32x2 nope[2][8];       // FP8: 8 codes per row piece
  u32x4 nope16[kFp8 ? 1 : 2][kFp8 ? 1 : 8];  // bf16 rows: 8 values per row piece
  u32x4 rope[2];
  float scale;
};

__device__ __forceinline__ int row_of_pos(int p) {
  // inverse of vt_pos
  const int rh = p >> 5, kap = (p >> 4) & 1, hf = (p >> 3) & 1, e = p & 7;
  return 32 * rh + 16 * kap + (e < 4 ? 4 * hf + e : 8 + 4 * hf + (e - 4));
}

template <bool kFp8>
__device__ __forceinline__ void gather_load(TileRegs<kFp8>& tr, const uint8_t* __restrict__ kv,
                                            const int32_t* rid) {
  constexpr int kRow = kFp8 ? kFp8Row : kBf16Row;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int g = tid + kDecThreads * it;
    const int dg = g & 63, rg = g >> 6;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int32_t r = rid[row_of_pos(8 * rg + e)];
      if constexpr (kFp8) {
        tr.nope[it][e] = u32x2{0u, 0u};
        if (r >= 0) tr.nope[it][e] = *reinterpret_cast<const u32x2*>(kv + (int64_t)r * kRow + 8 * dg);
      } else {
        tr.nope16[it][e] = u32x4{0u, 0u, 0u, 0u};
        if (r >= 0) tr.nope16[it][e] = *reinterpret_cast<const u32x4*>(kv + (int64_t)r * kRow + 16 * dg);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int c = tid + kDecThreads * it;
    const int row = c >> 3, part = c & 7;
    const int32_t r = rid[row];
    tr.rope[it] = u32x4{0u, 0u, 0u, 0u};
    if (r >= 0)
      tr.rope[it] = *reinterpret_cast<const u32x4*>(kv + (int64_t)r * kRow + (kFp8 ? 512 : 1024) + 16 * part);
  }
  tr.scale = 0.0f;
  if (kFp8 && tid < kTileRows) {
    const int32_t r = rid[tid];
    if (r >= 0) tr.scale = *reinterpret_cast<const float*>(kv + (int64_t)r * kRow + 640);
  }
}

// Convert and store a gathered tile: K row-major (bf16, 576 per row) and V^T (bf16, dim-major,
// rows in transposed-position order).
template <bool kFp8>
__device__ __forceinline__ void gather_store(const TileRegs<kFp8>& tr, unsigned char* lds) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int g = tid + kDecThreads * it;
    const int dg = g & 63, rg = g >> 6;
    u32x4 v[8];  // 8 rows x 8 bf16 values (dims 8 dg .. 8 dg + 7)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (kFp8) {
        v[e] = __builtin_bit_cast(u32x4, e4m3x8_to_bf16(tr.nope[it][e][0], tr.nope[it][e][1]));
      } else {
        v[e] = tr.nope16[it][e];
      }
      const int row = row_of_pos(8 * rg + e);
      *reinterpret_cast<u32x4*>(lds + row * DecLds::kKStride + 16 * dg) = v[e];
    }
    // transpose the 8 x 8 block of 16-bit values: dim d gets rows (positions) 0..7
    unsigned char* vt = lds + DecLds::kOffVt + 2 * 8 * rg;
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
      *reinterpret_cast<u32x4*>(vt + (8 * dg + 2 * dw) * DecLds::kVtStride) = even;
      *reinterpret_cast<u32x4*>(vt + (8 * dg + 2 * dw + 1) * DecLds::kVtStride) = odd;
    }
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int c = tid + kDecThreads * it;
    const int row = c >> 3, part = c & 7;
    *reinterpret_cast<u32x4*>(lds + row * DecLds::kKStride + 1024 + 16 * part) = tr.rope[it];
  }
  if (tid < kTileRows) reinterpret_cast<float*>(lds + DecLds::kOffScale)[tid] = kFp8 ? tr.scale : 1.0f;
}

template <bool kFp8>
__global__ __launch_bounds__(kDecThreads) void sparse_mla_decode_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ row_ids,
    const int32_t* __restrict__ ctx_lens, int B, int S, int K, int max_ctx,
    const uint8_t* __restrict__ kv, int64_t n_rows_pool, float qk_scale_log2, int splits,
    int xcd_map, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, int32_t* __restrict__ err) {
  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int32_t rid_next[kTileRows];
  // probabilities of each wave's row half, in its PV operand layout: [hg][dh][kap][lane]
  __shared__ __align__(16) u32x4 pshare[2][2][2][64];
  __shared__ float mshare[2][2][32];  // per-tile row maximum of each half, per head
  __shared__ float lshare[2][2][32];  // final row sums

  // Workgroup -> (request, query, split).  With xcd_map, the S*splits workgroups of a request
  // get ids congruent mod 8, i.e. the same XCD (workgroups are dealt to XCDs round-robin), so
  // the MTP queries of a request, which select mostly the same rows, share its L2.
  const int per_req = S * splits;
  int b, r;
  if (xcd_map) {
    const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
    b = xcd + 8 * (slot / per_req);
    r = slot % per_req;
  } else {
    b = blockIdx.x / per_req;
    r = blockIdx.x % per_req;
  }
  const int j = r / splits, sp = r % splits;
  const int bj = b * S + j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // head group hg: heads 32 hg .. 32 hg + 31.  dh: this wave scores tile rows 32 dh .. 32 dh + 31
  // and accumulates value dims 256 dh .. 256 dh + 255 over all rows.
  const int hg = wave & 1, dh = wave >> 1;
  const int col = lane & 31, hf = lane >> 5;
  const int head = 32 * hg + col;

  const int Lb = ctx_lens[b];
  int n = 0;
  if (Lb >= S && Lb <= max_ctx) n = min(K, Lb - S + 1 + j);
  else if (tid == 0 && sp == 0) raise_error(err, HS_DEVERR_SHORT_CONTEXT);
  const int per = ((n + splits - 1) / splits + kTileRows - 1) / kTileRows * kTileRows;
  const int r0 = sp * per, r1 = min(n, r0 + per);
  const int32_t* rids = row_ids + (int64_t)bj * K;

  // Q^T fragments (B operand): k-step s covers dims 16 s .. 16 s + 15, lane half hf holds
  // 8 hf .. 8 hf + 7 of them, for head `head`.
  bf16x8 qf[36];
  {
    const uint16_t* qp = q + ((int64_t)bj * kHeads + head) * kDqk + 8 * hf;
#pragma unroll
    for (int s = 0; s < 36; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
  }

  f32x16 o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f32x16{};
  float m_used = -INFINITY, l_part = 0.0f;

  // row ids of a tile: validated copy in LDS (bad or missing rows read as zero)
  auto load_rids = [&](int t0) {
    if (tid < kTileRows) {
      const int i = t0 + tid;
      int32_t v = -1;
      if (i < r1) {
        v = rids[i];
        if (v < 0 || v >= n_rows_pool) {
          raise_error(err, HS_DEVERR_BAD_ROW);
          v = -1;
        }
      }
      rid_next[tid] = v;
    }
  };

  const float* scale = reinterpret_cast<const float*>(lds + DecLds::kOffScale);
  for (int t0 = r0; t0 < r1; t0 += kTileRows) {
    const int n_tile = min(kTileRows, r1 - t0);
    __syncthreads();  // the previous tile's LDS reads are done
    load_rids(t0);
    __syncthreads();
    {
      TileRegs<kFp8> tr;
      gather_load<kFp8>(tr, kv, rid_next);
      gather_store<kFp8>(tr, lds);
    }
    __syncthreads();

    // ---- S^T = K Q^T for rows 32 dh .. +31 and this wave's 32 heads
    const unsigned char* kp = lds + (32 * dh + col) * DecLds::kKStride + 16 * hf;
    f32x16 c = {};
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + 32 * s));
      c = mfma32x32x16(a, qf[s], c);
      if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound how far reads are hoisted
    }
    // nope part times the row's scale, then the rope part accumulates on top
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] *= scale[32 * dh + 8 * (i >> 2) + 4 * hf + (i & 3)];
#pragma unroll
    for (int s = 32; s < 36; ++s) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + 32 * s));
      c = mfma32x32x16(a, qf[s], c);
    }
    // ---- online softmax: lane owns head `head`; rows 8(i/4) + 4 hf + i%4 of its half
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = 32 * dh + 8 * (i >> 2) + 4 * hf + (i & 3);
      // rows past the range and skipped rows (id -1) are left out of the softmax
      c[i] = rr < n_tile && rid_next[rr] >= 0 ? c[i] * qk_scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, c[i]);
    }
    {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if (hf == 0) mshare[hg][dh][col] = tmax;
    __syncthreads();
    tmax = fmaxf(tmax, mshare[hg][dh ^ 1][col]);  // the tile maximum over both halves
    if (tmax > m_used + kLazyRescale) {  // same decision in both waves of the head group
      const float alpha = exp2f(m_used - tmax);
      l_part *= alpha;
#pragma unroll
      for (int m = 0; m < 8; ++m) o[m] *= alpha;
      m_used = tmax;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // masked rows give 0, also before any row was seen (m_used = -inf)
      const float p = c[i] > -INFINITY ? exp2f(c[i] - m_used) : 0.0f;
      l_part += p;
      const float a = scale[32 * dh + 8 * (i >> 2) + 4 * hf + (i & 3)];
      pb[i >> 3][i & 7] = (__bf16)(p * a);
    }
    pshare[hg][dh][0][lane] = __builtin_bit_cast(u32x4, pb[0]);
    pshare[hg][dh][1][lane] = __builtin_bit_cast(u32x4, pb[1]);
    __syncthreads();
    // ---- O^T += V^T P^T over all 64 rows (4 k-steps of 16) for dims 256 dh .. +255
    const unsigned char* vp =
        lds + DecLds::kOffVt + (256 * dh + col) * DecLds::kVtStride + 2 * (8 * hf);
#pragma unroll
    for (int half_rows = 0; half_rows < 2; ++half_rows) {
#pragma unroll
      for (int kap = 0; kap < 2; ++kap) {
        const bf16x8 bp = half_rows == dh ? pb[kap]
                                          : __builtin_bit_cast(bf16x8, pshare[hg][half_rows][kap][lane]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              vp + 32 * m * DecLds::kVtStride + 2 * (32 * half_rows + 16 * kap)));
          o[m] = mfma32x32x16(a, bp, o[m]);
          if ((m & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // ---- finish: the row sums of both halves, then output (or split partial)
  float l_half;
  {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
    l_half = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  __syncthreads();
  if (hf == 0) lshare[hg][dh][col] = l_half;
  __syncthreads();
  const float l_tot = l_half + lshare[hg][dh ^ 1][col];
  if (splits == 1) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* op = out + ((int64_t)bj * kHeads + head) * kDv + 256 * dh;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const __bf16 v0 = (__bf16)(o[m][4 * g4 + 0] * inv), v1 = (__bf16)(o[m][4 * g4 + 1] * inv);
        const __bf16 v2 = (__bf16)(o[m][4 * g4 + 2] * inv), v3 = (__bf16)(o[m][4 * g4 + 3] * inv);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *reinterpret_cast<u32x2*>(op + 32 * m + 8 * g4 + 4 * hf) = u32x2{w0, w1};
      }
    if (lse && hf == 0 && dh == 0)
      lse[(int64_t)bj * kHeads + head] = (m_used + log2f(l_tot)) * 0.69314718055994531f;
  } else {
    const int64_t part = (int64_t)bj * splits + sp;
    if (hf == 0 && dh == 0) {
      part_ml[(part * kHeads + head) * 2 + 0] = m_used;
      part_ml[(part * kHeads + head) * 2 + 1] = l_tot;
    }
    if (r1 > r0) {
      float* pp = part_o + (part * kHeads + head) * kDv + 256 * dh;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(pp + 32 * m + 8 * g4 + 4 * hf) =
              f32x4{o[m][4 * g4], o[m][4 * g4 + 1], o[m][4 * g4 + 2], o[m][4 * g4 + 3]};
    }
  }
}

// ---------------------------------------------------------------------------------------
// FP8 rows: tiles stay FP8 in LDS.
//
// A tile is fetched by direct global->LDS loads (16 bytes per lane; rows keep their stored
// 656-byte pitch) one tile ahead of the tile being computed, so no registers hold rows in
// flight.  QK over the 512 nope dims runs on the FP8 codes as stored (16x16x128 FP8 MFMAs, 32
// bytes of a row per lane), the bf16 query carried by two E4M3 parts with per-head power-of-two
// scales that together keep its 8 significant bits (set up once per workgroup); the 64 rope dims
// stay bf16.  V^T is read with the transposing 8-byte read (ds_read_b64_tr_b8: in each group of
// 16 lanes, lanes 2k and 2k+1 address the two halves of a 16-byte segment of "row" k and lane r
// receives byte r of all eight segments), which hands a lane the 8 rows of one value dim that its
// MFMA k-slots take, and converted to bf16 exactly for the PV product (the probabilities stay
// bf16: their FP8 parts would need scales per 32 rows, which the output layout of QK does not
// group).  The rows behind the k-slots are addressed in the order the probabilities come out of
// the QK result, so nothing is permuted in memory.
//
// Work split (the waves specialise): score wave hb (0..3) holds Q for heads 16 hb .. +15 over
// all 576 dims and scores all 64 rows of a tile, so it alone decides its heads' running maxima
// (no exchange between waves) and writes the probabilities to LDS, already in the PV B-operand
// layout (the QK result of lane (head, g) is exactly the P fragment of that lane for that head
// block and 32-row k-step), with the factor by which the tile rescales O.  Value wave pw (0..3)
// accumulates O^T for value dims 128 pw .. +127 of all 64 heads, so each FP8 value of a tile is
// converted once.  The two kinds work on consecutive tiles through a ring of three tile buffers
// (being loaded, being scored, being accumulated), so each SIMD holds one wave of each and their
// MFMA and VALU work overlaps; one barrier per tile.  The score waves issue the tile loads (the
// value waves hold the larger register state: O is 128 registers).  Each role runs a loop of its
// own, so a wave keeps only its own role's registers, under 256, and two waves share each SIMD.
constexpr int kF8RowChunks = kFp8Row / 16;                   // 41 pieces of 16 bytes per row
constexpr int kF8TileBytes = kTileRows * kFp8Row;            // 41,984
constexpr int kF8TileLoads = kTileRows * kF8RowChunks / 64;  // 41 wave-wide loads per tile
static_assert(kTileRows * kF8RowChunks % 64 == 0, "whole wave-wide loads per tile");
static_assert(kF8RowChunks == 41 && kTileRows * kF8RowChunks <= 2688, "division by 41 below");

// Within the 32 16-byte pieces of a row's FP8 codes, rows with bit 4 set keep piece c at
// position c ^ 8.  With the 656-byte pitch, rows r and r + 16 otherwise start on the same LDS
// bank, and the transposed V reads take rows r and r + 16 together; the swap moves the second
// onto the 32 banks the first leaves free.  (An involution: the same map finds a piece's
// position and a position's piece.)
__device__ __forceinline__ int nope_swizzle(int piece, int row) {
  return piece < 32 ? piece ^ (8 * ((row >> 4) & 1)) : piece;
}

typedef int lds_i32x2 __attribute__((vector_size(8)));

__device__ __forceinline__ u32x2 lds_read_tr8(const unsigned char* p) {
  const lds_i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) lds_i32x2*)(p));
  return u32x2{(uint32_t)v[0], (uint32_t)v[1]};
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four floats (|x| < 448) -> their OCP E4M3 codes, rounded to nearest even, one per byte
// (element e in byte e); *v gets the values the codes stand for.
__device__ __forceinline__ uint32_t pack_e4m3x4(const float* x, float* v) {
  i16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[0], x[1], 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[2], x[3], 1.0f, true);
  const uint32_t code = (uint32_t)__builtin_bit_cast(int, w);
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)code, 1.0f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)code, 1.0f, true);
  v[0] = lo[0];
  v[1] = lo[1];
  v[2] = hi[0];
  v[3] = hi[1];
  return code;
}

// C += A B^T-style 16x16x128 product of E4M3 operands, B scaled by 2^(scale_b - 127) (one
// E8M0 scale per column of B).  Lane l holds A[l%16][32(l/16) .. +32] and B[32(l/16) .. +32][l%16],
// byte j of its eight dwords being element j; c[i] = C[4(l/16)+i][l%16].
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(const i32x8& a, const i32x8& b, int scale_b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

constexpr int kF8Threads = 512;  // 8 waves: 4 score waves (QK + softmax), 4 value waves (PV)
constexpr int kF8Bufs = 3;       // tile ring: scored, accumulated, loading
constexpr float kNoMax = -1.0e30f;  // running maximum before any row (finite: exp2 of it is 0)

__global__ __launch_bounds__(kF8Threads) void sparse_mla_decode_fp8_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ row_ids,
    const int32_t* __restrict__ ctx_lens, int B, int S, int K, int max_ctx,
    const uint8_t* __restrict__ kv, int64_t n_rows_pool, float qk_scale_log2, int splits,
    int xcd_map, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml, const uint8_t* __restrict__ zero_row, int32_t* __restrict__ err) {
  // the tile ring (distinct objects: one being loaded, one scored, one accumulated)
  __shared__ __align__(16) unsigned char tiles[kF8Bufs][kF8TileBytes];
  __shared__ __align__(16) int32_t rids[kMaxTopk];        // this workgroup's row ids (-1: skipped)
  __shared__ __align__(16) float bias[kMaxTopk];          // 0 for a row in the softmax, -inf otherwise
  __shared__ __align__(16) bf16x8 pls[2][2][4][64];       // P fragments: [tile parity][k-step][head block][lane]
  __shared__ float alph[2][kHeads];                       // rescale of O before the tile, per head
  __shared__ float lsum[kHeads];                          // final row sum per head
  // The tiles are written only by the asm loads: hand their addresses to asm so that the
  // compiler does not take them for never-written memory.
  asm volatile("" : : "v"(tiles) : "memory");

  const int per_req = S * splits;
  int b, r;
  if (xcd_map) {
    const int slot = blockIdx.x / 8;
    b = (blockIdx.x % 8) + 8 * (slot / per_req);
    r = slot % per_req;
  } else {
    b = blockIdx.x / per_req;
    r = blockIdx.x % per_req;
  }
  const int j = r / splits, sp = r % splits;
  const int bj = b * S + j;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Score wave hb (0..3): heads 16 hb .. +15 over all 64 rows of a tile.  Value wave pw (0..3):
  // value dims 128 pw .. +127 of all 64 heads.  In the 16x16 MFMA layouts lane l works on head
  // (16 x block) + l%16 and on rows / dims in groups of 4 selected by l/16.
  const bool scorer = wave < 4;
  const int hb = wave & 3, pw = wave & 3;
  const int c16 = lane & 15, g = lane >> 4;
  const int head = 16 * hb + c16;

  const int Lb = ctx_lens[b];
  int n = 0;
  if (Lb >= S && Lb <= max_ctx) n = min(K, Lb - S + 1 + j);
  else if (tid == 0 && sp == 0) raise_error(err, HS_DEVERR_SHORT_CONTEXT);
  const int per = ((n + splits - 1) / splits + kTileRows - 1) / kTileRows * kTileRows;
  const int r0 = min(n, sp * per), r1 = min(n, r0 + per);
  const int nrows = r1 - r0;
  const int ntiles = (nrows + kTileRows - 1) / kTileRows;

  // staged up to a whole tile (-1 past the range), so tile loads read them without bounds
  for (int i = tid; i < ntiles * kTileRows; i += kF8Threads) {
    int32_t v = -1;
    if (i < nrows) {
      v = row_ids[(int64_t)bj * K + r0 + i];
      if (v < 0 || v >= n_rows_pool) {
        raise_error(err, HS_DEVERR_BAD_ROW);
        v = -1;
      }
    }
    rids[i] = v;
    bias[i] = v >= 0 ? 0.0f : -INFINITY;
  }
  // Score waves: Q^T for the nope dims as the B operand of four FP8 k-steps of 128 dims (lane
  // group g holds dims 32 g .. +31 of the step for head `head`).  Each bf16 value q is carried by
  // two E4M3 parts: q 2^E = hi + lo / 16, with one power of two E per head and k-step that puts
  // the largest |q| in [128, 256).  hi keeps 4 significant bits, lo the next 4 of the remainder
  // (|remainder| <= half a step of hi), so hi + lo / 16 carries bf16's 8; the MFMA's per-column
  // E8M0 scales undo 2^E and the 16.  The rope dims stay bf16: two k-steps of 32, lane group g
  // holding 8 of each.
  i32x8 qh[4], ql[4];
  int q_sh[4];
  bf16x8 q_rope[2];
  if (scorer) {
    const uint16_t* qp = q + ((int64_t)bj * kHeads + head) * kDqk;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint16_t* p = qp + 128 * ks + 32 * g;
      float x[32];
      float m = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p + 8 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * v + 2 * e] = __uint_as_float(w[e] << 16);
          x[8 * v + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(x[e]));
      m = fmaxf(m, __shfl_xor(m, 16));  // the head's maximum over the four lane groups
      m = fmaxf(m, __shfl_xor(m, 32));
      int E = 0;
      if (m > 0.0f) E = 7 - ((int)((__float_as_uint(m) >> 23) & 255) - 127);
      E = max(-120, min(E, 120));
      const float sc = __builtin_ldexpf(1.0f, E);
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float xs[4], hv[4], rr[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xs[e] = x[4 * w + e] * sc;
        qh[ks][w] = (int)pack_e4m3x4(xs, hv);
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = (xs[e] - hv[e]) * 16.0f;  // exact: |xs - hv| <= half a step
        ql[ks][w] = (int)pack_e4m3x4(rr, lv);
      }
      q_sh[ks] = 127 - E;  // the lo part's scale is 2^-4 of it
    }
#pragma unroll
    for (int kr = 0; kr < 2; ++kr)
      q_rope[kr] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 512 + 32 * kr + 8 * g));
  }
  // Value waves: O^T[value dim 128 pw + 16 db + 4 g + i][head 16 hg + c16] in o[db][hg][i]
  f32x4 o[8][4];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) o[db][hg] = f32x4{};
  float m_qk = kNoMax, l_part = 0.0f;  // score waves: running maximum of `head`, partial row sum
  // Q and the row ids are in before any tile load is issued, and the compiler knows it: its
  // waits for them would otherwise sit inside the tile loop and also drain the prefetch.  (The
  // empty asm takes the fragments, so their loads cannot sink below this point.)
  if (scorer) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qh[ks]), "+v"(ql[ks]));
    asm volatile("" : "+v"(q_rope[0]), "+v"(q_rope[1]));
  }
  wait_vmcnt<0>();
  asm volatile("" ::: "memory");
  __syncthreads();  // row ids staged

  // Loads of tile rows [t0, t0 + 64) of the range into LDS address `buf`: wave-wide load ins
  // covers the 64 consecutive 16-byte pieces ins*64 .. ins*64+63 of the tile; wave w issues
  // w, w+8, ...  The row ids are read together before the first load is issued.
  // The score waves issue the tile loads (the value waves hold the larger register state).
  // Lane work of those loads, the same for every tile: wave-wide load i of score wave hb covers
  // the 64 consecutive 16-byte pieces (4 i + hb) * 64 .. +63 of the tile (rows of 41 pieces);
  // lane l takes the piece at position c = (4 i + hb) * 64 + l: row c / 41, stored at its
  // swizzled place in the row.
  constexpr int kLoaders = 4;
  constexpr int kPer = (kF8TileLoads + kLoaders - 1) / kLoaders;
  int row_l[kPer], off_l[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = min(kLoaders * i + hb, kF8TileLoads - 1) * 64 + lane;
    row_l[i] = (c * 1599) >> 16;  // c / 41 for c < 2,688
    off_l[i] = 16 * nope_swizzle(c - row_l[i] * kF8RowChunks, row_l[i]);
  }
  // Loads of tile rows [t0, t0 + 64) of the range into LDS address `buf`; the row ids are read
  // together before the first load is issued.  A skipped row (id -1: past the range, or
  // flagged) reads a row of zeros, so whatever the pool holds elsewhere cannot reach the
  // products; its logit is masked as well.
  auto issue = [&](uint32_t buf, int t0) {
    int32_t rid_l[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) rid_l[i] = rids[t0 + row_l[i]];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ins = kLoaders * i + hb;
      if (ins < kF8TileLoads) {
        const uint8_t* row = rid_l[i] >= 0 ? kv + (int64_t)rid_l[i] * kFp8Row : zero_row;
        lds_load16(row + off_l[i], buf + ins * 1024);
      }
    }
  };

  // ---- score wave: S^T = K Q^T for rows 16 mb + 4 g + i of the tile, head `head` (the nope
  // part on the FP8 codes as stored, times the row's scale, plus the rope part); the tile's
  // maximum per head, the lazy rescale, P (times the row scale) as the B operands of the two PV
  // k-steps, and the rescale factor the value waves apply before accumulating this tile
  auto score = [&](const unsigned char* buf, int t0, int par) {
    f32x4 c[4], rsc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) c[mb] = f32x4{};
    // k-step by k-step over the four row blocks, so that consecutive MFMAs are independent
    // and each k-step's key fragments are read while the previous k-step runs
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      i32x8 k8[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // rows of odd blocks have bit 4 set: their pieces 8 ks + 2 g (+1) sit 8 pieces away
        const int kss = (mb & 1) ? (ks ^ 1) : ks;
        const unsigned char* kp = buf + (16 * mb + c16) * kFp8Row + 32 * g + 128 * kss;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kp);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kp + 16);
        k8[mb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) c[mb] = mfma_f8_16x16x128(k8[mb], qh[ks], q_sh[ks], c[mb]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) c[mb] = mfma_f8_16x16x128(k8[mb], ql[ks], q_sh[ks] - 4, c[mb]);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int row0 = 16 * mb + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) rsc[mb][i] = *reinterpret_cast<const float*>(buf + (row0 + i) * kFp8Row + 640);
      c[mb] *= rsc[mb];
    }
#pragma unroll
    for (int kr = 0; kr < 2; ++kr)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const unsigned char* rp = buf + (16 * mb + c16) * kFp8Row + 512 + 64 * kr + 16 * g;
        c[mb] = mfma16x16x32(as_bf16x8(*reinterpret_cast<const u32x4*>(rp)), q_rope[kr], c[mb]);
      }
    // logits in log2 units; rows outside the softmax get -inf from their bias, so their
    // probabilities below are exactly 0
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const f32x4 bs = *reinterpret_cast<const f32x4*>(&bias[t0 + 16 * mb + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[mb][i] = __builtin_fmaf(c[mb][i], qk_scale_log2, bs[i]);
        tmax = fmaxf(tmax, c[mb][i]);
      }
    }
    {  // the head's maximum over the four lane groups
      auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // the running maximum only moves when it grows by more than 2^kLazyRescale (v_exp_f32:
    // results below 2^-126 flush to 0, far below what a sum of probabilities <= 2^kLazyRescale
    // can notice)
    float alpha = 1.0f;
    if (tmax > m_qk + kLazyRescale) {
      alpha = __builtin_amdgcn_exp2f(m_qk - tmax);
      l_part *= alpha;
      m_qk = tmax;
    }
    if (g == 0) alph[par][head] = alpha;
    // k-step kk of the PV product: k-slot 8g + e holds row 32 kk + 4g + e (e < 4) or
    // 32 kk + 16 + 4g + e - 4, i.e. blocks 2 kk and 2 kk + 1 of this lane
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 pb;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mb = 2 * kk + h;
          const float p = __builtin_amdgcn_exp2f(c[mb][i] - m_qk);
          l_part += p;
          pb[4 * h + i] = (__bf16)(p * rsc[mb][i]);
        }
      pls[par][kk][hb][lane] = pb;
    }
  };

  // Transposed V reads of a value wave: lane group g takes the k-slots 8g .. 8g+7 of a 32-row
  // k-step, which hold the rows the P fragments put there (rows 4g .. 4g+3 and 16+4g .. 16+4g+3
  // of the step).  The wave's value dims 128 pw + 16 db .. +15 are piece 8 pw + db; rows 16+ of
  // a step (kk8 >= 4) have it at piece (8 pw + db) ^ 8, i.e. 128 bytes later when pw is even
  // and 128 bytes earlier when it is odd.
  const int kk8 = (lane & 15) >> 1;
  const int v_lane_off = (kk8 < 4 ? 4 * g + kk8 : 16 + 4 * g + (kk8 - 4)) * kFp8Row + 128 * pw + 8 * (lane & 1) +
                         (kk8 >= 4 ? ((pw & 1) ? -128 : 128) : 0);

  // ---- value wave: O^T = alpha O^T + V^T P^T over the tile's two k-steps of 32 rows
  auto accumulate = [&](const unsigned char* buf, int par) {
    float a[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) a[hg] = alph[par][16 * hg + c16];
    if (__builtin_amdgcn_ballot_w64(a[0] != 1.0f || a[1] != 1.0f || a[2] != 1.0f || a[3] != 1.0f)) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int hg = 0; hg < 4; ++hg)
          o[db][hg] *= a[hg];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const unsigned char* vp = buf + 32 * kk * kFp8Row + v_lane_off;
      bf16x8 pv[4];
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) pv[hg] = pls[par][kk][hg][lane];
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const u32x2 raw = lds_read_tr8(vp + 16 * db);
        const bf16x8 va = e4m3x8_to_bf16(raw[0], raw[1]);
#pragma unroll
        for (int hg = 0; hg < 4; ++hg)
          o[db][hg] = mfma16x16x32(va, pv[hg], o[db][hg]);
      }
    }
  };

  // Tile i lives in ring buffer i % 3.  Round k: after every wave has seen tile k land (and so
  // has finished round k - 1), tile k + 1 is loaded into the buffer tile k - 2 used, the score
  // waves score tile k while the value waves accumulate tile k - 1 (scored in round k - 1), so
  // the two kinds of work share each SIMD.  One barrier per round; the two roles run loops of
  // their own (the same number of rounds and barriers), so each keeps only its own registers.
  auto ring = [&](int i) -> unsigned char* { return tiles[i]; };
  if (scorer) {
    if (ntiles > 0) issue(lds_address(tiles[0]), 0);
    for (int k = 0; k <= ntiles; ++k) {
      wait_vmcnt<0>();  // this wave's loads of tile k have landed
      lds_barrier();    // ... and every other wave's; round k - 1 is done everywhere
      if (k + 1 < ntiles) issue(lds_address(ring((k + 1) % kF8Bufs)), (k + 1) * kTileRows);
      if (k < ntiles) score(ring(k % kF8Bufs), k * kTileRows, k & 1);
    }
  } else {
    for (int k = 0; k <= ntiles; ++k) {
      lds_barrier();
      if (k >= 1) accumulate(ring((k - 1) % kF8Bufs), (k - 1) & 1);
    }
  }

  // ---- finish: the score waves hold each head's running maximum and row sum (over the four
  // lane groups); the value waves normalise
  if (scorer) {
    float l = l_part;
    auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (g == 0) {
      lsum[head] = l;
      if (splits == 1) {
        if (lse) lse[(int64_t)bj * kHeads + head] = (m_qk + log2f(l)) * 0.69314718055994531f;
      } else {
        const int64_t part = (int64_t)bj * splits + sp;
        part_ml[(part * kHeads + head) * 2 + 0] = m_qk;
        part_ml[(part * kHeads + head) * 2 + 1] = l;
      }
    }
  }
  __syncthreads();
  if (scorer) return;
  if (splits == 1) {
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const float l_tot = lsum[16 * hg + c16];
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      uint16_t* op = out + ((int64_t)bj * kHeads + 16 * hg + c16) * kDv + 128 * pw + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const __bf16 v0 = (__bf16)(o[db][hg][0] * inv), v1 = (__bf16)(o[db][hg][1] * inv);
        const __bf16 v2 = (__bf16)(o[db][hg][2] * inv), v3 = (__bf16)(o[db][hg][3] * inv);
        const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *reinterpret_cast<u32x2*>(op + 16 * db) = u32x2{w0, w1};
      }
    }
  } else if (nrows > 0) {
    const int64_t part = (int64_t)bj * splits + sp;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      float* pp = part_o + (part * kHeads + 16 * hg + c16) * kDv + 128 * pw + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(pp + 16 * db) = o[db][hg];
    }
  }
}

// Combine the split partials of each query: M = max m_s, L = sum l_s 2^(m_s - M),
// out = sum O_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.  Workgroup = (query, kH heads), 512
// threads: each of a head's 128 pieces of 4 value dims is summed by kG threads, each over its
// share of the splits (at most kPer), with all of a thread's loads issued before the first use;
// the kG sums meet in LDS.  Many splits (few queries): one head per workgroup and 4 groups, so
// that a lone query still spreads over 64 workgroups; few splits: 4 heads and one group, so
// that a large batch does not launch a workgroup per head.
constexpr int kMergeThreads = 512;
constexpr int kMergePieces = kDv / 4;  // 128

template <int kH, int kG, int kPer>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float* __restrict__ part_o,
                                                                     const float* __restrict__ part_ml,
                                                                     int splits, uint16_t* __restrict__ out,
                                                                     float* __restrict__ lse) {
  static_assert(kH * kG * kMergePieces == kMergeThreads && kG * kPer >= 1 && kG * kPer <= 64, "shape");
  __shared__ float fac[kH][kG * kPer];  // 2^(m_s - M), 0 for an empty split
  __shared__ float inv_l[kH];
  __shared__ f32x4 gsum[kG > 1 ? kG - 1 : 1][kH][kMergePieces];
  const int bj = blockIdx.x / (kHeads / kH), h0 = (blockIdx.x % (kHeads / kH)) * kH;
  const int tid = threadIdx.x;
  if (tid < 64) {  // wave 0: the factors of each head, one split per lane
#pragma unroll
    for (int hl = 0; hl < kH; ++hl) {
      float m = -INFINITY, l = 0.0f;
      if (tid < splits) {
        const float* ml = part_ml + (((int64_t)bj * splits + tid) * kHeads + h0 + hl) * 2;
        m = ml[0];
        l = ml[1];
      }
      const float M = wave_max(l > 0.0f ? m : -INFINITY);
      const float f = l > 0.0f ? exp2f(m - M) : 0.0f;
      float L = l * f;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
      if (tid < kG * kPer) fac[hl][tid] = f;
      if (tid == 0) {
        inv_l[hl] = L > 0.0f ? 1.0f / L : 0.0f;
        if (lse) lse[(int64_t)bj * kHeads + h0 + hl] = (M + log2f(L)) * 0.69314718055994531f;
      }
    }
  }
  __syncthreads();
  const int piece = tid % kMergePieces, hl = (tid / kMergePieces) % kH, grp = tid / (kMergePieces * kH);
  // Buffer loads relative to this query's partials: a split past the last gets an offset past
  // the end, which reads zero without a memory access, so every load is an unconditional
  // instruction and all of them are issued before the first use.
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(part_o + (int64_t)bj * splits * kHeads * kDv), (short)0,
      splits * kHeads * kDv * (int)sizeof(float), kBufferRsrcWord3);
  f32x4 v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int sp = grp + kG * k;
    const int off = sp < splits ? ((sp * kHeads + h0 + hl) * kDv + 4 * piece) * (int)sizeof(float) : (int)0x80000000;
    v[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 0));
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int sp = grp + kG * k;  // < kG * kPer
    // an empty split's partial was never written: dropped by the select, not scaled by 0
    const float f = sp < splits ? fac[hl][sp] : 0.0f;
    acc += f != 0.0f ? v[k] * f : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (kG > 1) {
    if (grp > 0) gsum[grp - 1][hl][piece] = acc;
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int g = 0; g < kG - 1; ++g) acc += gsum[g][hl][piece];
  }
  const float inv = inv_l[hl];
  const __bf16 v0 = (__bf16)(acc[0] * inv), v1 = (__bf16)(acc[1] * inv);
  const __bf16 v2 = (__bf16)(acc[2] * inv), v3 = (__bf16)(acc[3] * inv);
  const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
  const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
  *reinterpret_cast<u32x2*>(out + ((int64_t)bj * kHeads + h0 + hl) * kDv + 4 * piece) = u32x2{w0, w1};
}

// Row ids of a prefill chunk's selections: queries [0, n) of the chunk, query i seeing
// `visible0 + i` rows; token t of the request reads row block_table[t / 64] * 64 + t % 64 (a
// prefill reads resident pages: a placeholder page flags HS_DEVERR_BAD_BLOCK).  Without a
// top-K (topk == nullptr) query i takes every row it sees, as a prompt within top-K does.
__global__ void prefill_rows_kernel(const int32_t* __restrict__ topk, int K, int n, int visible0,
                                    const int32_t* __restrict__ bt, int n_pages,
                                    int64_t num_gpu_blocks, int32_t* __restrict__ rows,
                                    int32_t* __restrict__ err) {
  const int64_t total = (int64_t)n * K;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx / K), k = (int)(idx - (int64_t)i * K);
    const int visible = visible0 + i;
    const int32_t t = topk ? topk[idx] : (k < visible ? k : -1);
    int32_t r = -1;
    if (t >= visible || (t >= 0 && (t >> 6) >= n_pages)) {
      raise_error(err, HS_DEVERR_BAD_ROW);
    } else if (t >= 0) {
      const int32_t blk = bt[t >> 6];
      if (blk >= 0 && blk < num_gpu_blocks) r = blk * kBlock + (t & 63);
      else raise_error(err, HS_DEVERR_BAD_BLOCK);
    }
    rows[idx] = r;
  }
}

}  // namespace

// Fixed scratch of sparse_mla_decode_noalloc, for callers that cannot allocate: the split-K
// partials of up to kFixedPartials (query, split) pairs, the outputs [kFixedPartials][64][512]
// fp32 first, then the (max, sum) pairs [kFixedPartials][64][2].  Host code never passes the
// array's name to a kernel: it takes the device address from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[(size_t)kFixedPartials * kHeads * (kDv + 2) * 4];

}  // namespace hs

using namespace hs;

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[hs::kMaxDevices] = {};
}  // namespace

hipError_t hs_fixed_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(hs::scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

void* hs_fixed_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

size_t hs_decode_lds_bytes(int) { return DecLds::kTotal; }

int hs_choose_splits(const hs_ctx* ctx, int B, int S) {
  // enough workgroups for one per CU (one workgroup fills a CU's LDS)
  const int nq = B * S;
  const int tiles = (ctx->cfg.topk + kTileRows - 1) / kTileRows;
  int splits = (256 + nq - 1) / nq;
  if (splits > tiles) splits = tiles;
  if (splits > ctx->lay.splits_cap) splits = ctx->lay.splits_cap;
  if (splits < 1) splits = 1;
  return splits;
}

hipError_t hs_launch_decode(const hs_ctx* ctx, int layer, const void* q, const int32_t* row_ids,
                            const int32_t* ctx_lens, int B, int S, float sm_scale, void* out,
                            float* lse, int splits, hipStream_t stream, float* part_o,
                            float* part_ml) {
  if (!part_o) part_o = ctx->ws.part_o;
  if (!part_ml) part_ml = ctx->ws.part_ml;
  const hs_config& c = ctx->cfg;
  const int64_t n_rows_pool = c.num_gpu_blocks * kBlock;
  const uint8_t* kv = static_cast<const uint8_t*>(ctx->buf.kv_pool) +
                      (int64_t)layer * n_rows_pool * ctx->row_bytes;
  const float qk_scale_log2 = sm_scale * 1.4426950408889634f;
  const int xcd_map = (B % 8 == 0) ? 1 : 0;
  const dim3 grid((unsigned)(B * S * splits));
  hs_timer_mark(ctx, HS_KERNEL_DECODE, true, stream);
  if (c.kv_dtype == HS_FP8_E4M3)
    hipLaunchKernelGGL(sparse_mla_decode_fp8_kernel, grid, dim3(kF8Threads), 0, stream,
                       static_cast<const uint16_t*>(q), row_ids, ctx_lens, B, S, c.topk,
                       c.max_pages_per_req * kBlock, kv, n_rows_pool, qk_scale_log2, splits,
                       xcd_map, static_cast<uint16_t*>(out), lse, part_o, part_ml,
                       ctx->ws.zero_row, ctx->ws.err);
  else
    hipLaunchKernelGGL(sparse_mla_decode_kernel<false>, grid, dim3(kDecThreads), DecLds::kTotal, stream,
                       static_cast<const uint16_t*>(q), row_ids, ctx_lens, B, S, c.topk,
                       c.max_pages_per_req * kBlock, kv, n_rows_pool, qk_scale_log2, splits,
                       xcd_map, static_cast<uint16_t*>(out), lse, part_o, part_ml,
                       ctx->ws.err);
  hs_timer_mark(ctx, HS_KERNEL_DECODE, false, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hs_timer_mark(ctx, HS_KERNEL_DECODE_MERGE, true, stream);
  static_assert(kMaxSplits == 32, "merge shapes below cover up to 32 splits");
  if (splits > 8)
    hipLaunchKernelGGL((decode_merge_kernel<1, 4, 8>), dim3((unsigned)(B * S * kHeads)), dim3(kMergeThreads), 0,
                       stream, part_o, part_ml, splits, static_cast<uint16_t*>(out), lse);
  else if (splits > 2)
    hipLaunchKernelGGL((decode_merge_kernel<4, 1, 8>), dim3((unsigned)(B * S * kHeads / 4)), dim3(kMergeThreads), 0,
                       stream, part_o, part_ml, splits, static_cast<uint16_t*>(out), lse);
  else
    hipLaunchKernelGGL((decode_merge_kernel<4, 1, 2>), dim3((unsigned)(B * S * kHeads / 4)), dim3(kMergeThreads), 0,
                       stream, part_o, part_ml, splits, static_cast<uint16_t*>(out), lse);
  hs_timer_mark(ctx, HS_KERNEL_DECODE_MERGE, false, stream);
  return hipGetLastError();
}

// Raise the dynamic-LDS limit of the bf16-row decode kernel.
hipError_t hs_set_kernel_attributes() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_mla_decode_kernel<false>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, DecLds::kTotal);
}

// Prefill attention on the sparse-MLA decode kernel: the P new tokens of request b, in chunks of
// max_batch x max_queries queries run as decode-shaped groups (see hs_launch_prefill_lens).
hipError_t hs_launch_prefill_decode(const hs_ctx* ctx, int layer, int b, const void* q,
                                    const int32_t* topk, int L, int P, float sm_scale, void* out,
                                    float* lse, hipStream_t stream) {
  const hs_config& c = ctx->cfg;
  const int S = c.max_queries, chunk = c.max_batch * c.max_queries, K = c.topk;
  const int32_t* bt = ctx->buf.block_table + (int64_t)b * c.max_pages_per_req;
  const size_t q_bytes = (size_t)kHeads * kDqk * 2, o_bytes = (size_t)kHeads * kDv * 2;
  for (int c0 = 0; c0 < P; c0 += chunk) {
    const int n = P - c0 < chunk ? P - c0 : chunk;
    const int full = n / S, rem = n - full * S;
    hipError_t e = hs_launch_prefill_lens(ctx, L, P, c0, n, stream);
    if (e != hipSuccess) return e;
    const int64_t cells = (int64_t)n * K;
    int blocks = (int)((cells + 255) / 256);
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(prefill_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       topk ? topk + (int64_t)c0 * K : nullptr, K, n, L - P + 1 + c0, bt,
                       c.max_pages_per_req, (int64_t)c.num_gpu_blocks, ctx->ws.pf_rows, ctx->ws.err);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned char* qb = static_cast<const unsigned char*>(q) + (size_t)c0 * q_bytes;
    unsigned char* ob = static_cast<unsigned char*>(out) + (size_t)c0 * o_bytes;
    float* lb = lse ? lse + (int64_t)c0 * kHeads : nullptr;
    if (full) {
      e = hs_launch_decode(ctx, layer, qb, ctx->ws.pf_rows, ctx->ws.pf_lens, full, S, sm_scale, ob,
                           lb, hs_choose_splits(ctx, full, S), stream);
      if (e != hipSuccess) return e;
    }
    if (rem) {
      const int i0 = full * S;
      e = hs_launch_decode(ctx, layer, qb + (size_t)i0 * q_bytes, ctx->ws.pf_rows + (int64_t)i0 * K,
                           ctx->ws.pf_lens + full, 1, rem, sm_scale, ob + (size_t)i0 * o_bytes,
                           lb ? lb + (int64_t)i0 * kHeads : nullptr, hs_choose_splits(ctx, 1, rem),
                           stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}
