/*
 * Seeded synthetic inputs for the quantized decode path.
 *
 * This file draws random numbers and writes them into buffers.  It does none
 * of the method's arithmetic: it never decodes a block, never forms a weight
 * value and never touches an activation.  The only format knowledge here is
 * where each field sits in a block (so that a scale lands in the scale field)
 * and the block sizes, which both the checker and the GPU library read back.
 *
 * Generator: counter-based SplitMix64.  Every tensor is a "stream" named by
 * (seed, stream id); value i of a stream is mix(key + (i + 1) * GOLDEN), with
 * key = mix(mix(seed) ^ stream).  mix() is Steele, Lea and Flood's SplitMix64
 * finalizer (OOPSLA 2014).  Being counter-based, any chunk of a tensor can be
 * produced on any thread, and any single block can be regenerated alone.
 *
 * Block layouts written here (little-endian, fp16 = IEEE binary16):
 *   Q8_0  34 B / 32 weights : d fp16 @0, q int8[32] @2
 *   Q4_0  18 B / 32 weights : d fp16 @0, packed nibbles[16] @2
 *   Q4_K 144 B / 256 weights: d fp16 @0, dmin fp16 @2, packed 6-bit scales[12] @4, nibbles[128] @16
 *   Q6_K 210 B / 256 weights: low nibbles[128] @0, high 2-bit fields[64] @128, int8 scales[16] @192, d fp16 @208
 *   Q5_K 176 B / 256 weights: d fp16 @0, dmin fp16 @2, packed 6-bit scales[12] @4, high bits[32] @16, nibbles[128] @48
 * Packed bit fields are filled with uniform random bytes, which makes every
 * field (4-bit, 6-bit, 2-bit) uniform over its full range, as the workloads ask.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ stream);
}

/* value number i of the stream keyed by key */
static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* uniform double in [0, 1) from the top 53 bits */
static inline double u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

/* Round a double to the nearest IEEE binary16 value, ties to even.  Used to
 * store scales and cache entries drawn in double precision. */
uint16_t synth_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u; /* at or past the rounding point to +inf */
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  int E = e - 1; /* a = 1.f * 2^E */
  if (E < -14) E = -14; /* subnormal range: fixed quantum 2^-24 */
  double quantum = ldexp(1.0, E - 10);
  double n = nearbyint(a / quantum); /* exact division by a power of two, RNE rounding */
  if (n < 1024.0) return sign | (uint16_t)n; /* subnormal or zero */
  if (n >= 2048.0) { n *= 0.5; E += 1; }
  if (E + 15 >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)(((E + 15) << 10) | ((uint32_t)n - 1024u));
}

static inline void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

static inline uint16_t scale_f16(uint64_t w, double lo, double hi) { return synth_f64_to_f16(lo + (hi - lo) * u01(w)); }

/* fill n bytes starting at value counter c0 (8 bytes per draw) */
static inline void fill_bytes(uint8_t* p, int n, uint64_t key, uint64_t c0) {
  for (int i = 0; i < n; i += 8) {
    uint64_t w = draw(key, c0 + (uint64_t)(i / 8));
    int m = n - i < 8 ? n - i : 8;
    for (int j = 0; j < m; ++j) p[i + j] = (uint8_t)(w >> (8 * j));
  }
}

/* Each block owns a fixed window of 32 counters, so block b is the same
 * whatever range of blocks a call fills. */
#define BLOCK_COUNTERS 32ULL

/* Q8_0: d ~ U[dlo, dhi] rounded to fp16; q ~ U{-127..127} (multiply-shift of a
 * 32-bit draw onto 255 values; bias below 2^-24). */
void synth_fill_q8_0(uint8_t* out, int64_t b0, int64_t nb, uint64_t seed, uint64_t stream, double dlo, double dhi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nb; ++i) {
    uint64_t c = (uint64_t)(b0 + i) * BLOCK_COUNTERS;
    uint8_t* blk = out + i * 34;
    put_u16(blk, scale_f16(draw(key, c), dlo, dhi));
    for (int j = 0; j < 32; j += 2) {
      uint64_t w = draw(key, c + 1 + (uint64_t)(j / 2));
      for (int h = 0; h < 2; ++h) {
        uint64_t u = (w >> (32 * h)) & 0xFFFFFFFFULL;
        int q = (int)((u * 255ULL) >> 32) - 127;
        blk[2 + j + h] = (uint8_t)(int8_t)q;
      }
    }
  }
}

/* Q4_0: d ~ U[dlo, dhi] fp16; nibbles uniform. */
void synth_fill_q4_0(uint8_t* out, int64_t b0, int64_t nb, uint64_t seed, uint64_t stream, double dlo, double dhi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nb; ++i) {
    uint64_t c = (uint64_t)(b0 + i) * BLOCK_COUNTERS;
    uint8_t* blk = out + i * 18;
    put_u16(blk, scale_f16(draw(key, c), dlo, dhi));
    fill_bytes(blk + 2, 16, key, c + 1);
  }
}

/* Q4_K: d, dmin ~ U[dlo, dhi] fp16; 6-bit scales/mins and nibbles uniform. */
void synth_fill_q4_k(uint8_t* out, int64_t b0, int64_t nb, uint64_t seed, uint64_t stream, double dlo, double dhi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nb; ++i) {
    uint64_t c = (uint64_t)(b0 + i) * BLOCK_COUNTERS;
    uint8_t* blk = out + i * 144;
    put_u16(blk + 0, scale_f16(draw(key, c), dlo, dhi));
    put_u16(blk + 2, scale_f16(draw(key, c + 1), dlo, dhi));
    fill_bytes(blk + 4, 140, key, c + 2); /* 12 scale bytes + 128 nibble bytes */
  }
}

/* Q5_K: d, dmin ~ U[dlo, dhi] fp16; 6-bit scales/mins, high bits and nibbles uniform. */
void synth_fill_q5_k(uint8_t* out, int64_t b0, int64_t nb, uint64_t seed, uint64_t stream, double dlo, double dhi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nb; ++i) {
    uint64_t c = (uint64_t)(b0 + i) * BLOCK_COUNTERS;
    uint8_t* blk = out + i * 176;
    put_u16(blk + 0, scale_f16(draw(key, c), dlo, dhi));
    put_u16(blk + 2, scale_f16(draw(key, c + 1), dlo, dhi));
    fill_bytes(blk + 4, 172, key, c + 2); /* 12 scale bytes + 32 high-bit bytes + 128 nibble bytes */
  }
}

/* Q6_K: d ~ U[dlo, dhi] fp16; int8 sub-scales ~ U{-64..63}; 6-bit codes uniform. */
void synth_fill_q6_k(uint8_t* out, int64_t b0, int64_t nb, uint64_t seed, uint64_t stream, double dlo, double dhi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nb; ++i) {
    uint64_t c = (uint64_t)(b0 + i) * BLOCK_COUNTERS;
    uint8_t* blk = out + i * 210;
    fill_bytes(blk, 192, key, c + 1); /* low nibbles + high bit pairs */
    uint8_t s[16];
    fill_bytes(s, 16, key, c + 25);
    for (int j = 0; j < 16; ++j) blk[192 + j] = (uint8_t)(int8_t)((int)(s[j] & 0x7F) - 64);
    put_u16(blk + 208, scale_f16(draw(key, c), dlo, dhi));
  }
}

/* Standard normal pairs by Box-Muller (one draw pair per two outputs). */
static inline void normal_pair(uint64_t key, uint64_t i, double* a, double* b) {
  double u1 = u01(draw(key, 2 * i));
  double u2 = u01(draw(key, 2 * i + 1));
  double r = sqrt(-2.0 * log(1.0 - u1)); /* 1 - u1 in (0, 1] */
  double t = 6.283185307179586476925286766559 * u2;
  *a = r * cos(t);
  *b = r * sin(t);
}

/* out[k] for k in [e0, e0 + n) of the stream: N(mean, std) rounded to fp32 */
void synth_fill_normal_f32(float* out, int64_t e0, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) {
    double a, b;
    int64_t e = e0 + k;
    normal_pair(key, (uint64_t)(e / 2), &a, &b);
    out[k] = (float)(mean + std * ((e & 1) ? b : a));
  }
}

/* N(mean, std) rounded to fp16 bits */
void synth_fill_normal_f16(uint16_t* out, int64_t e0, int64_t n, uint64_t seed, uint64_t stream, double mean, double std) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) {
    double a, b;
    int64_t e = e0 + k;
    normal_pair(key, (uint64_t)(e / 2), &a, &b);
    out[k] = synth_f64_to_f16(mean + std * ((e & 1) ? b : a));
  }
}

/* U[lo, hi] rounded to fp32 */
void synth_fill_uniform_f32(float* out, int64_t e0, int64_t n, uint64_t seed, uint64_t stream, double lo, double hi) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < n; ++k) out[k] = (float)(lo + (hi - lo) * u01(draw(key, (uint64_t)(e0 + k))));
}

/* uniform integer in [0, n) by multiply-shift of a 32-bit draw */
int64_t synth_uniform_index(uint64_t seed, uint64_t stream, int64_t n) {
  uint64_t w = draw(stream_key(seed, stream), 0) >> 32;
  return (int64_t)((w * (uint64_t)n) >> 32);
}

/* raw 64-bit draws, for tests of the generator itself */
void synth_raw(uint64_t* out, int64_t c0, int64_t n, uint64_t seed, uint64_t stream) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, (uint64_t)(c0 + i));
}
