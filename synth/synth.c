/*
 * Seeded synthetic inputs for the Hybrid HiSparse sparse-MLA decode step.
 *
 * This module only produces input bytes.  It holds none of the method's
 * arithmetic (no scoring, selection, residency logic or attention); both the
 * CPU oracle and the GPU harness read what it writes.
 *
 * Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), keyed by (seed, kind) with a 128-bit
 * counter (i/4, a, b, c).  Every value is therefore addressable on its own:
 * any token's key or latent row can be regenerated without the others.
 * Normal variates use the Box-Muller transform (single precision libm).
 *
 * Storage formats written here:
 *   bf16            round-to-nearest-even from fp32.
 *   OCP FP8 E4M3FN  round-to-nearest-even, saturating at +-448, subnormals
 *                   kept (exponent bias 7, no infinities, 0x7F/0xFF = NaN,
 *                   never produced).
 *   FP8 indexer key 128 e4m3 codes with one fp32 per-token scale
 *                   (scale = amax / 448), the 132-byte-per-token indexer
 *                   layout of the GLM-5.3 part-2 page, footnote 3.
 *   FP8 latent row  656 bytes: [0,512) e4m3 "nope" codes scaled by one fp32
 *                   per-token scale, [512,640) 64 bf16 rope values, [640,644)
 *                   the fp32 scale, [644,656) zero.  The pages give only the
 *                   656-byte total (part-2 page, footnote 1); this split is
 *                   the reading adopted for it.
 *   bf16 latent row 576 bf16 values (1152 bytes).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define SY_EXPORT __attribute__((visibility("default")))

/* ---------------------------------------------------------------- Philox */

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

static inline void philox4x32_10(const uint32_t ctr[4], uint32_t seed, uint32_t kind,
                                 uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {seed, kind};
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k);
    k[0] += 0x9E3779B9u;
    k[1] += 0xBB67AE85u;
  }
  out[0] = c[0];
  out[1] = c[1];
  out[2] = c[2];
  out[3] = c[3];
}

/* uniform in the open interval (0, 1) with 24 random bits */
static inline double u01(uint32_t x) { return ((double)(x >> 8) + 0.5) * (1.0 / 16777216.0); }

/* four N(0,1) variates for counter (blk, a, b, c); Box-Muller in single precision */
static inline void normal4(uint32_t seed, uint32_t kind, uint32_t blk, uint32_t a, uint32_t b,
                           uint32_t c, float z[4]) {
  uint32_t ctr[4] = {blk, a, b, c}, r[4];
  philox4x32_10(ctr, seed, kind, r);
  const float two_pi = 6.28318530717958647692f;
  float r0 = sqrtf(-2.0f * logf((float)u01(r[0])));
  float r1 = sqrtf(-2.0f * logf((float)u01(r[2])));
  float s0, c0, s1, c1;
  sincosf(two_pi * (float)u01(r[1]), &s0, &c0);
  sincosf(two_pi * (float)u01(r[3]), &s1, &c1);
  z[0] = r0 * c0;
  z[1] = r0 * s0;
  z[2] = r1 * c1;
  z[3] = r1 * s1;
}

/* n consecutive normals of stream (kind; a, b, c), element i uses block i/4 */
static void normals(uint32_t seed, uint32_t kind, uint32_t a, uint32_t b, uint32_t c, int n,
                    float* out) {
  float z[4];
  for (int i = 0; i < n; i += 4) {
    normal4(seed, kind, (uint32_t)(i / 4), a, b, c, z);
    for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = z[j];
  }
}

/* ------------------------------------------------------------ encoders */

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  x += 0x7FFFu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

/* OCP E4M3FN, round to nearest even, saturate to the largest finite (448) */
static inline uint8_t f32_to_e4m3_rne_sat(float f) {
  uint8_t sign = (f < 0.0f || (f == 0.0f && signbit(f))) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (!(a < 464.0)) return (uint8_t)(sign | 0x7E); /* >= 448 + half ulp, or NaN */
  if (a < 0.015625) {                              /* below 2^-6: subnormal grid 2^-9 */
    double m = nearbyint(a * 512.0);               /* 0..8; 8 is the smallest normal */
    return (uint8_t)(sign | (uint8_t)m);
  }
  int ex;
  double fr = frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
  int e = ex - 1;            /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
  double m = nearbyint((2.0 * fr - 1.0) * 8.0);
  if (m >= 8.0) {
    m = 0.0;
    e += 1;
  }
  int E = e + 7;
  if (E > 15 || (E == 15 && m > 6.0)) return (uint8_t)(sign | 0x7E);
  return (uint8_t)(sign | (uint8_t)(E << 3) | (uint8_t)m);
}

SY_EXPORT uint16_t synth_bf16_from_f32(float f) { return f32_to_bf16_rne(f); }
SY_EXPORT uint8_t synth_e4m3_from_f32(float f) { return f32_to_e4m3_rne_sat(f); }

SY_EXPORT void synth_encode_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(in[i]);
}

SY_EXPORT void synth_encode_e4m3(const float* in, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_e4m3_rne_sat(in[i]);
}

/* quantise v[0..n) as e4m3 with one fp32 scale = amax/448 (scale 1 if all zero) */
static float quant_e4m3_row(const float* v, int n, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  for (int i = 0; i < n; ++i) codes[i] = f32_to_e4m3_rne_sat(v[i] / scale);
  return scale;
}

/* ------------------------------------------------------------ streams */

enum {
  KIND_IDX_KEY = 1,  /* (b, t)          indexer key, 128 normals */
  KIND_SALIENT = 2,  /* (b, t)          salience draw, one uniform */
  KIND_LATENT = 3,   /* (b, t, layer)   latent row, 576 normals */
  KIND_QIDX0 = 4,    /* (b)             indexer query chain start, 4096 normals */
  KIND_QIDX_EPS = 5, /* (b, n)          indexer query chain innovation */
  KIND_W = 6,        /* (b, j)          indexer head weights, 32 uniforms */
  KIND_Q = 7,        /* (b, n)          MLA query, 64 x 576 normals */
  KIND_UNIFORM = 8   /* (a, b, c)       generic uniforms for recipes */
};

SY_EXPORT void synth_philox(uint32_t seed, uint32_t kind, uint32_t c0, uint32_t c1, uint32_t c2,
                            uint32_t c3, uint32_t* out4) {
  uint32_t ctr[4] = {c0, c1, c2, c3};
  philox4x32_10(ctr, seed, kind, out4);
}

SY_EXPORT void synth_normals(uint32_t seed, uint32_t kind, uint32_t a, uint32_t b, uint32_t c,
                             int32_t n, float* out) {
  normals(seed, kind, a, b, c, n, out);
}

/* n uniforms in (0,1) of stream (kind; a, b, c): element i uses word i%4 of block i/4 */
SY_EXPORT void synth_uniforms(uint32_t seed, uint32_t kind, uint32_t a, uint32_t b, uint32_t c,
                              int32_t n, double* out) {
  for (int i = 0; i < n; i += 4) {
    uint32_t ctr[4] = {(uint32_t)(i / 4), a, b, c}, r[4];
    philox4x32_10(ctr, seed, kind, r);
    for (int j = 0; j < 4 && i + j < n; ++j) out[i + j] = u01(r[j]);
  }
}

/* Is token t of request b salient?  Bernoulli(frac), fixed across steps. */
static inline int is_salient(uint32_t seed, int32_t b, int64_t t, double frac) {
  uint32_t ctr[4] = {0u, (uint32_t)b, (uint32_t)t, 0u}, r[4];
  philox4x32_10(ctr, seed, KIND_SALIENT, r);
  return u01(r[0]) < frac;
}

SY_EXPORT void synth_salient_mask(uint32_t seed, int32_t b, int64_t t0, int64_t n, double frac,
                                  uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)is_salient(seed, b, t0 + i, frac);
}

/* The fp32 indexer key of token t (before storage rounding): N(0, I), plus
 * `shift` on every component when the token is salient. */
static void idx_key_f32(uint32_t seed, int32_t b, int64_t t, double frac, float shift,
                        float k[128]) {
  normals(seed, KIND_IDX_KEY, (uint32_t)b, (uint32_t)t, 0u, 128, k);
  if (frac > 0.0 && is_salient(seed, b, t, frac))
    for (int d = 0; d < 128; ++d) k[d] += shift;
}

/*
 * Indexer keys of whole pages of request b, written into a paged pool.
 *   page_ids[i]   logical page of the request (tokens 64*page .. +64)
 *   dst_block[i]  destination block in `pool`
 *   idx_dtype 0 (bf16): block = 64 x 128 bf16 = 16384 bytes
 *   idx_dtype 1 (fp8) : block = 64 x 128 e4m3 codes, then 64 fp32 scales = 8448 bytes
 */
SY_EXPORT void synth_idx_pages(uint32_t seed, int32_t idx_dtype, int32_t b, int64_t n_pages,
                               const int32_t* page_ids, const int64_t* dst_block, uint8_t* pool,
                               double salient_frac, float salient_shift) {
  const int64_t blk_bytes = idx_dtype == 0 ? 16384 : 8448;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < n_pages * 64; ++i) {
    const int64_t p = i / 64, o = i % 64;
    const int64_t t = (int64_t)page_ids[p] * 64 + o;
    uint8_t* blk = pool + dst_block[p] * blk_bytes;
    float k[128];
    idx_key_f32(seed, b, t, salient_frac, salient_shift, k);
    if (idx_dtype == 0) {
      uint16_t* dst = (uint16_t*)(blk + o * 256);
      for (int d = 0; d < 128; ++d) dst[d] = f32_to_bf16_rne(k[d]);
    } else {
      float scale = quant_e4m3_row(k, 128, blk + o * 128);
      memcpy(blk + 8192 + o * 4, &scale, 4);
    }
  }
}

/* Indexer keys of tokens [t0, t0+n) in token order (not paged), for checkers:
 *   bf16: out_codes holds n*256 bytes; fp8: n*128 codes plus n fp32 scales. */
SY_EXPORT void synth_idx_tokens(uint32_t seed, int32_t idx_dtype, int32_t b, int64_t t0, int64_t n,
                                uint8_t* out_codes, float* out_scale, double salient_frac,
                                float salient_shift) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float k[128];
    idx_key_f32(seed, b, t0 + i, salient_frac, salient_shift, k);
    if (idx_dtype == 0) {
      uint16_t* dst = (uint16_t*)(out_codes + i * 256);
      for (int d = 0; d < 128; ++d) dst[d] = f32_to_bf16_rne(k[d]);
    } else {
      out_scale[i] = quant_e4m3_row(k, 128, out_codes + i * 128);
    }
  }
}

/* One stored latent row of (b, layer, t). kv_dtype 0: 1152 bytes; 1: 656 bytes. */
static void latent_row(uint32_t seed, int32_t kv_dtype, int32_t b, int32_t layer, int64_t t,
                       uint8_t* dst) {
  float v[576];
  normals(seed, KIND_LATENT, (uint32_t)b, (uint32_t)t, (uint32_t)layer, 576, v);
  if (kv_dtype == 0) {
    uint16_t* d16 = (uint16_t*)dst;
    for (int d = 0; d < 576; ++d) d16[d] = f32_to_bf16_rne(v[d]);
  } else {
    float scale = quant_e4m3_row(v, 512, dst);
    uint16_t* rope = (uint16_t*)(dst + 512);
    for (int d = 0; d < 64; ++d) rope[d] = f32_to_bf16_rne(v[512 + d]);
    memcpy(dst + 640, &scale, 4);
    memset(dst + 644, 0, 12);
  }
}

/*
 * Latent rows of whole pages of (b, layer) into a row-addressed buffer:
 * token 64*page_ids[i] + o goes to row dst_row0[i] + o of `dst` (row_bytes apart).
 */
SY_EXPORT void synth_latent_pages(uint32_t seed, int32_t kv_dtype, int32_t b, int32_t layer,
                                  int64_t n_pages, const int32_t* page_ids,
                                  const int64_t* dst_row0, uint8_t* dst) {
  const int64_t rb = kv_dtype == 0 ? 1152 : 656;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < n_pages * 64; ++i) {
    const int64_t p = i / 64, o = i % 64;
    latent_row(seed, kv_dtype, b, layer, (int64_t)page_ids[p] * 64 + o, dst + (dst_row0[p] + o) * rb);
  }
}

/* Latent rows of an arbitrary token list, packed (row i = tokens[i]). */
SY_EXPORT void synth_latent_tokens(uint32_t seed, int32_t kv_dtype, int32_t b, int32_t layer,
                                   int64_t n, const int64_t* tokens, uint8_t* out) {
  const int64_t rb = kv_dtype == 0 ? 1152 : 656;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) latent_row(seed, kv_dtype, b, layer, tokens[i], out + i * rb);
}

/*
 * Indexer query chain of request b over flattened query tokens n = 0..n_count-1:
 *   q_0 ~ N(0, I) (32 x 128), q_{n+1} = rho q_n + sigma eps_n, in fp32, then
 * stored as bf16.  Writes n_count x 4096 bf16 codes.
 */
SY_EXPORT void synth_qidx_chain(uint32_t seed, int32_t b, int32_t n_count, float rho, float sigma,
                                uint16_t* out) {
  float q[4096], eps[4096];
  normals(seed, KIND_QIDX0, (uint32_t)b, 0u, 0u, 4096, q);
  for (int n = 0; n < n_count; ++n) {
    if (n > 0) {
      normals(seed, KIND_QIDX_EPS, (uint32_t)b, (uint32_t)(n - 1), 0u, 4096, eps);
      for (int i = 0; i < 4096; ++i) q[i] = rho * q[i] + sigma * eps[i];
    }
    for (int i = 0; i < 4096; ++i) out[(int64_t)n * 4096 + i] = f32_to_bf16_rne(q[i]);
  }
}

/* MLA queries of request b for flattened query tokens n0..n0+count: 64 x 576 bf16 each. */
SY_EXPORT void synth_mla_q(uint32_t seed, int32_t b, int32_t n0, int32_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < count; ++i) {
    float v[64 * 576];
    normals(seed, KIND_Q, (uint32_t)b, (uint32_t)(n0 + i), 0u, 64 * 576, v);
    for (int e = 0; e < 64 * 576; ++e) out[(int64_t)i * 64 * 576 + e] = f32_to_bf16_rne(v[e]);
  }
}

SY_EXPORT int32_t synth_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
