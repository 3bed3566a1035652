/*
 * CHECKER — test infrastructure only.  Plain, slow, obviously correct CPU
 * definition of what the quantized batch-1 decode path computes, in fp64.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this; the GPU library never does, and shares no code with it.
 *
 * Sources (the ntransformer pages):
 *  - ntransformer overview (de.news.hada.io), "Überblick über NTransformer":
 *    the engine reads GGUF weights in Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K, F16, F32.
 *  - same page, "Hauptfunktionen": Llama layers with RoPE, GQA, SwiGLU,
 *    RMSNorm and a KV cache; "Roadmap der Entwicklungsphasen": F16 KV cache.
 *  - same page, "Architektur und Codestruktur": GEMV, RMSNorm, RoPE, SwiGLU
 *    and softmax kernels; transformer, attention, FFN and norm in the model.
 *  - 70B PCIe P2P article (blog.hotdry.top), §传统数据路径的性能瓶颈分析: every
 *    generated token touches the whole weight set.
 * The pages do not print the block byte layouts.  This file decodes the
 * public GGML block layouts (the readings are listed in the design notes):
 *   Q8_0 (34 B / 32): d fp16 @0, q int8[32] @2;            w = d*q
 *   Q4_0 (18 B / 32): d fp16 @0, nibbles[16] @2;           w = d*(n-8), weight i<16 is the low
 *                      nibble of byte i, weight i>=16 the high nibble of byte i-16
 *   Q4_K (144 B / 256): d @0, dmin @2, scales[12] @4, nibbles[128] @16; w = d*sc_j*q - dmin*m_j
 *   Q5_K (176 B / 256): d @0, dmin @2, scales[12] @4 (packed as in Q4_K), high bits[32] @16,
 *                      nibbles[128] @48; q = nibble + 16 * (bit j of high byte i mod 32),
 *                      w = d*sc_j*q - dmin*m_j
 *   Q6_K (210 B / 256): low nibbles[128] @0, 2-bit highs[64] @128, int8 s[16] @192, d @208;
 *                      w = d*s_(i/16)*(q-32)
 *   F16 (2 B / 1), F32 (4 B / 1): the weight itself, IEEE binary16 / binary32 (GGUF's
 *                      unquantized tensor types, listed by the overview beside the quant formats)
 * With these fields every weight is an exact fp64 number (at most 32
 * significant bits), so dequantization to fp32 is a single RNE rounding of the
 * exact value, and every dot product here is accumulated in fp64.
 *
 * Parity pins: dequant (hand-built blocks, exhaustive scale packing sweep,
 * all codes); GEMV (exact-rational brute force, one-hot and constant inputs);
 * RMSNorm, RoPE, attention and SwiGLU (closed forms, invariants, library
 * routines on special cases).  See tests/test_oracle_pins.py.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_Q8_0 = 0, OR_Q4_0 = 1, OR_Q4_K = 2, OR_Q6_K = 3, OR_Q5_K = 4, OR_F16 = 5, OR_F32 = 6 };

/* Threads of the OpenMP loops below (for timing the checker on a stated core count). */
void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int or_get_threads(void) { return omp_get_max_threads(); }

int or_block_elems(int fmt) {
  switch (fmt) {
    case OR_Q8_0: case OR_Q4_0: return 32;
    case OR_Q4_K: case OR_Q6_K: case OR_Q5_K: return 256;
    case OR_F16: case OR_F32: return 1;  /* unquantized: one weight per "block" */
  }
  return -1;
}

int or_block_bytes(int fmt) {
  switch (fmt) {
    case OR_Q8_0: return 34;
    case OR_Q4_0: return 18;
    case OR_Q4_K: return 144;
    case OR_Q6_K: return 210;
    case OR_Q5_K: return 176;
    case OR_F16: return 2;
    case OR_F32: return 4;
  }
  return -1;
}

/* IEEE 754 binary16 -> fp64, from the definition: sign, 5-bit biased
 * exponent, 10-bit fraction.  Exact. */
double or_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1024.0 + (double)f, e - 25);            /* (1 + f/1024) * 2^(e-15) */
  return sign ? -v : v;
}

static double rd16(const uint8_t* p) { return or_f16((uint16_t)(p[0] | (p[1] << 8))); }

/* The two 6-bit numbers (scale, min) of sub-block j (0..7) of a Q4_K block.
 * Sub-blocks 0..3 keep them in the low 6 bits of bytes j and j+4; sub-blocks
 * 4..7 keep their low 4 bits in the two nibbles of byte j+4 and their top two
 * bits in the high bits of bytes j-4 (scale) and j (min). */
static void q4k_scale_min(const uint8_t* s, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
    *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

/* Exact value of every weight of one block, in fp64. */
static void dequant_block(int fmt, const uint8_t* b, double* w) {
  switch (fmt) {
    case OR_F16:  /* IEEE binary16, little-endian */
      w[0] = rd16(b);
      break;
    case OR_F32: {  /* IEEE binary32, little-endian; every binary32 value is exact in fp64 */
      float f;
      memcpy(&f, b, 4);
      w[0] = (double)f;
      break;
    }
    case OR_Q8_0: {
      double d = rd16(b);
      for (int i = 0; i < 32; ++i) w[i] = d * (double)(int8_t)b[2 + i];
      break;
    }
    case OR_Q4_0: {
      double d = rd16(b);
      for (int i = 0; i < 32; ++i) {
        int n = i < 16 ? (b[2 + i] & 15) : (b[2 + i - 16] >> 4);
        w[i] = d * (double)(n - 8);
      }
      break;
    }
    case OR_Q4_K: {
      double d = rd16(b), dmin = rd16(b + 2);
      const uint8_t* sc = b + 4;
      const uint8_t* qs = b + 16;
      for (int i = 0; i < 256; ++i) {
        int j = i / 32, g = i / 64, l = i % 32;
        int q = (qs[32 * g + l] >> (4 * (j % 2))) & 15;
        int s, m;
        q4k_scale_min(sc, j, &s, &m);
        w[i] = d * (double)s * (double)q - dmin * (double)m;
      }
      break;
    }
    case OR_Q5_K: {
      /* as Q4_K, with a fifth code bit: weight i of sub-block j takes bit j of
       * high-bit byte i mod 32, worth 16 */
      double d = rd16(b), dmin = rd16(b + 2);
      const uint8_t* sc = b + 4;
      const uint8_t* qh = b + 16;
      const uint8_t* qs = b + 48;
      for (int i = 0; i < 256; ++i) {
        int j = i / 32, g = i / 64, l = i % 32;
        int q = ((qs[32 * g + l] >> (4 * (j % 2))) & 15) + 16 * ((qh[l] >> j) & 1);
        int s, m;
        q4k_scale_min(sc, j, &s, &m);
        w[i] = d * (double)s * (double)q - dmin * (double)m;
      }
      break;
    }
    case OR_Q6_K: {
      const uint8_t* ql = b;
      const uint8_t* qh = b + 128;
      const int8_t* s = (const int8_t*)(b + 192);
      double d = rd16(b + 208);
      for (int i = 0; i < 256; ++i) {
        int h = i / 128, r = i % 128, k = r / 32, l = r % 32;
        int lo = (ql[64 * h + 32 * (k % 2) + l] >> (4 * (k / 2))) & 15;
        int hi = (qh[32 * h + l] >> (2 * k)) & 3;
        int q = lo | (hi << 4);
        w[i] = d * (double)s[i / 16] * (double)(q - 32);
      }
      break;
    }
  }
}

/* One row (cols weights) of a row-major block matrix, exact in fp64. */
int or_dequant_row(int fmt, int64_t cols, const uint8_t* row, double* w) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  if (be < 0 || cols % be) return -1;
  for (int64_t k = 0; k < cols / be; ++k) dequant_block(fmt, row + k * bb, w + k * be);
  return 0;
}

/* Dequantized matrix, each weight rounded once (RNE) from its exact value to fp32. */
int or_dequant_f32(int fmt, int64_t rows, int64_t cols, const uint8_t* blocks, float* out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  if (be < 0 || cols % be) return -1;
  int64_t row_bytes = cols / be * bb;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      or_dequant_row(fmt, cols, blocks + r * row_bytes, w);
      for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = (float)w[c];
    }
    free(w);
  }
  return 0;
}

/* y_r = sum_c w_rc x_c with exact weights and fp64 sums; nrm_r = sum_c |w_rc x_c|.
 * row_idx (nullable) picks which rows to compute: output k is row row_idx[k];
 * with row_idx NULL, outputs 0..n_out-1 are rows 0..n_out-1. */
int or_gemv(int fmt, int64_t rows, int64_t cols, const uint8_t* blocks, const double* x, double* y,
            double* nrm, const int64_t* row_idx, int64_t n_out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  if (be < 0 || cols % be) return -1;
  int64_t row_bytes = cols / be * bb;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)cols);
#pragma omp for schedule(dynamic, 16)
    for (int64_t k = 0; k < n_out; ++k) {
      int64_t r = row_idx ? row_idx[k] : k;
      if (r < 0 || r >= rows) { y[k] = NAN; if (nrm) nrm[k] = NAN; continue; }
      or_dequant_row(fmt, cols, blocks + r * row_bytes, w);
      double s = 0.0, a = 0.0;
      for (int64_t c = 0; c < cols; ++c) {
        s += w[c] * x[c];
        a += fabs(w[c] * x[c]);
      }
      y[k] = s;
      if (nrm) nrm[k] = a;
    }
    free(w);
  }
  return 0;
}

/* RMSNorm: y_i = g_i * x_i / sqrt(mean(x^2) + eps), eps inside the root. */
void or_rmsnorm(int64_t n, const double* x, const double* g, double eps, double* y) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) y[i] = g[i] * x[i] * inv;
}

/* RoPE on n_heads consecutive heads of head_dim values, in place.  Pair i of
 * a head is the adjacent pair (2i, 2i+1); its frequency is theta^(-2i/head_dim)
 * and it is turned by the angle pos * frequency. */
void or_rope(int n_heads, int head_dim, int64_t pos, double theta, double* x) {
  for (int h = 0; h < n_heads; ++h) {
    double* v = x + (int64_t)h * head_dim;
    for (int i = 0; i < head_dim / 2; ++i) {
      double f = pow(theta, -2.0 * (double)i / (double)head_dim);
      double a = (double)pos * f;
      double c = cos(a), s = sin(a);
      double x0 = v[2 * i], x1 = v[2 * i + 1];
      v[2 * i] = x0 * c - x1 * s;
      v[2 * i + 1] = x0 * s + x1 * c;
    }
  }
}

/* GQA decode attention for one new token.  q: [n_q][hd]; caches
 * [n_kv][max_ctx][hd] fp16 bits; query head h reads KV head h / (n_q / n_kv).
 * Scores s_t = q . k_t / sqrt(hd) for t in [0, n_ctx); p = softmax(s) with the
 * maximum subtracted; out_h = sum_t p_t v_t.  nrm (nullable) gets, per output
 * element, sum_t p_t |v_t[d]|. */
int or_attn(int n_q, int n_kv, int hd, int64_t n_ctx, int64_t max_ctx, const double* q,
            const uint16_t* kc, const uint16_t* vc, double* out, double* nrm) {
  if (n_kv <= 0 || n_q % n_kv || n_ctx <= 0 || n_ctx > max_ctx) return -1;
  int grp = n_q / n_kv;
  double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for schedule(dynamic, 1)
  for (int h = 0; h < n_q; ++h) {
    int g = h / grp;
    const double* qh = q + (int64_t)h * hd;
    double* s = (double*)malloc(sizeof(double) * (size_t)n_ctx);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n_ctx; ++t) {
      const uint16_t* kt = kc + ((int64_t)g * max_ctx + t) * hd;
      double acc = 0.0;
      for (int d = 0; d < hd; ++d) acc += qh[d] * or_f16(kt[d]);
      s[t] = acc * scale;
      if (s[t] > mx) mx = s[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < n_ctx; ++t) { s[t] = exp(s[t] - mx); z += s[t]; }
    for (int d = 0; d < hd; ++d) { out[(int64_t)h * hd + d] = 0.0; if (nrm) nrm[(int64_t)h * hd + d] = 0.0; }
    for (int64_t t = 0; t < n_ctx; ++t) {
      double p = s[t] / z;
      const uint16_t* vt = vc + ((int64_t)g * max_ctx + t) * hd;
      for (int d = 0; d < hd; ++d) {
        double v = or_f16(vt[d]);
        out[(int64_t)h * hd + d] += p * v;
        if (nrm) nrm[(int64_t)h * hd + d] += p * fabs(v);
      }
    }
    free(s);
  }
  return 0;
}

/* SwiGLU: a_i = silu(gate_i) * up_i with silu(g) = g / (1 + e^-g).
 * nrm (nullable) gets |gate_i| * |up_i|, a bound on |a_i| since the logistic is <= 1. */
void or_swiglu(int64_t n, const double* gate, const double* up, double* out, double* nrm) {
  for (int64_t i = 0; i < n; ++i) {
    double g = gate[i];
    double sig = g >= 0 ? 1.0 / (1.0 + exp(-g)) : exp(g) / (1.0 + exp(g));
    out[i] = g * sig * up[i];
    if (nrm) nrm[i] = fabs(g) * fabs(up[i]);
  }
}

/* fp64 -> nearest binary16 (ties to even), for the cache write. */
uint16_t or_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00u;
  if (a == 0.0) return sign;
  /* largest finite is 65504; halfway to the next binade step (65520) rounds up to inf */
  if (a >= 65520.0) return sign | 0x7C00u;
  int e = (int)floor(log2(a));
  if (ldexp(1.0, e) > a) e -= 1;          /* guard log2 rounding */
  if (ldexp(1.0, e + 1) <= a) e += 1;
  if (e < -14) e = -14;                   /* below the normal range the step is 2^-24 */
  double step = ldexp(1.0, e - 10);
  double k = a / step;                    /* exact: power-of-two division */
  double fl = floor(k), fr = k - fl;
  double n = fl;
  if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
  int64_t ni = (int64_t)n;
  if (ni < 1024) return sign | (uint16_t)ni;           /* subnormal */
  if (ni == 2048) { ni = 1024; e += 1; }
  if (e > 15) return sign | 0x7C00u;
  return sign | (uint16_t)(((e + 15) << 10) | (ni - 1024));
}

/* first index of the maximum (ties go to the lowest index) */
int64_t or_argmax(int64_t n, const double* v) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}
