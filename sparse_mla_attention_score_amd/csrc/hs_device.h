// Device helpers for gfx950: MFMA operand types, exact FP8 -> bf16, block-wide scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// C += A(32x16) * B(16x32): lane l supplies A[l%32][8(l/32)..+8] and B[8(l/32)..+8][l%32];
// c[i] is C[8(i/4) + 4(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C += A(16x32) * B(32x16): lane l supplies A[l%16][8(l/16)..+8] and B[8(l/16)..+8][l%16];
// c[i] is C[4(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight OCP E4M3 codes (byte k of the 64-bit pair = element k) -> eight bf16, exactly.
// Every E4M3 value, subnormals included, is representable in bf16; the scale is 1.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Byte permute of the 64-bit value {hi:lo}: selector byte k picks byte sel_k of it.
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Transpose a 4x4 byte block: in r0..r3 (row i = 4 bytes), out c0..c3 (column e = byte e of
// each row, row 0 in the low byte).
__device__ __forceinline__ void transpose4x4_bytes(uint32_t r0, uint32_t r1, uint32_t r2,
                                                   uint32_t r3, uint32_t& c0, uint32_t& c1,
                                                   uint32_t& c2, uint32_t& c3) {
  const uint32_t t01a = byte_perm(r1, r0, 0x05010400u);  // r0.b0 r1.b0 r0.b1 r1.b1
  const uint32_t t01b = byte_perm(r1, r0, 0x07030602u);  // r0.b2 r1.b2 r0.b3 r1.b3
  const uint32_t t23a = byte_perm(r3, r2, 0x05010400u);
  const uint32_t t23b = byte_perm(r3, r2, 0x07030602u);
  c0 = byte_perm(t23a, t01a, 0x05040100u);
  c1 = byte_perm(t23a, t01a, 0x07060302u);
  c2 = byte_perm(t23b, t01b, 0x05040100u);
  c3 = byte_perm(t23b, t01b, 0x07060302u);
}

// Transpose a 2x2 block of 16-bit values held as two dwords (row i = {lo16, hi16}).
__device__ __forceinline__ void transpose2x2_u16(uint32_t r0, uint32_t r1, uint32_t& c0,
                                                 uint32_t& c1) {
  c0 = byte_perm(r1, r0, 0x05040100u);  // r0.lo r1.lo
  c1 = byte_perm(r1, r0, 0x07060302u);  // r0.hi r1.hi
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits for this wave's LDS traffic only (not for loads in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One wave-wide direct load: lane l's 16 bytes at `src` land at LDS byte address lds + 16 l.
// Issued from asm on purpose: the compiler does not see these loads, so it adds no waits for
// them in front of LDS reads it cannot prove disjoint (e.g. the transposing reads); the
// kernel waits for them itself (wait_vmcnt, which only ever waits for more than the
// compiler's own bookkeeping would, as vector-memory operations complete in order).  No other
// instruction of the kernel uses m0.
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory");
}

// One wave-wide direct 4-byte load: lane l's 4 bytes at `src` land at LDS byte address lds + 4 l
// (inactive lanes write nothing).
__device__ __forceinline__ void lds_load4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(lds) : "memory");
}

// s_waitcnt lgkmcnt(0) alone: this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Exclusive prefix sum over a block of NT threads.  `scratch` holds NT/64 + 1 ints.
// Returns this thread's exclusive prefix; *total gets the block sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  static_assert(NT % 64 == 0 && NT <= 4096, "block size");
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = lane < kWaves ? scratch[lane] : 0;
    int u = t;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const int y = __shfl_up(u, o);
      if (lane >= o) u += y;
    }
    if (lane < kWaves) scratch[lane] = u - t;
    if (lane == kWaves - 1) scratch[kWaves] = u;
  }
  __syncthreads();
  const int res = scratch[wave] + x - v;
  *total = scratch[kWaves];
  __syncthreads();
  return res;
}

__device__ __forceinline__ void raise_error(int32_t* err, int32_t bit) {
  atomicOr(reinterpret_cast<int*>(err), bit);
}

// Word 3 of a raw buffer resource on gfx950 (32-bit data format, no swizzle, no index
// stride): offsets at or past num_records read as zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace hs
