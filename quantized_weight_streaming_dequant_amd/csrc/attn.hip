// GQA decode attention over an fp16 KV cache, one new token, gfx950 (MFMA).
//
// The pages' layer has GQA attention over a KV cache kept in fp16 (ntransformer
// overview, de.news.hada.io, "Hauptfunktionen" and "Roadmap der
// Entwicklungsphasen"), with a softmax kernel ("Architektur und Codestruktur").
//
// Both products of one KV head's group are small dense contractions, so they run on
// the matrix cores (v_mfma_f32_16x16x32_f16) while keeping fp32-level accuracy:
//  * scores S = K Q^T: K rows are exact fp16.  Each query head's row, pre-scaled by
//    log2(e)/sqrt(128) and by a power of two that brings its largest entry to
//    [2^13, 2^14), is split into hi = fp16(x) and lo = fp16(x - hi) (|x - hi - lo| is
//    about 2^-22 |x|); hi parts fill columns 0-7 of the 16-column operand, lo parts
//    columns 8-15, and the two columns of a head are summed after the MFMA.
//  * p V: p (in exp2 units, max-subtracted) is scaled by 2^12 and split the same way
//    into two fp16 rows per head; V is exact fp16; the rows are summed afterwards.
// Products of fp16 values are exact in fp32, so the error is the fp32 accumulation
// plus the ~2^-22 split residue, far inside the 1e-3 budget.
//
// Layout: K cache [n_kv][max_ctx][128] (row per slot); V cache in groups of 8 slots,
// [n_kv][max_ctx/8][128][8], so that one 16-byte load gives a lane the 8 consecutive
// slots of one dimension that the B operand of p V wants.
//
// Work split: workgroup (split, kv head) covers 256 slots, each of its eight waves 32.
// A wave's two 16-slot score tiles map MFMA row r to slot 8(r/4) + 4 tile + r%4, so
// that the output layout (lane l: rows 4(l/16)..+3, column l%16) leaves each lane
// the eight consecutive slots 8(l/16)..+7 of its column: exactly its A operand for
// p V, with no data movement.  The eight waves merge through LDS into one (max, sum,
// unnormalised output) partial per head; a second kernel merges the splits.  With a
// single split the first kernel writes the normalised output itself.
#include "attn.h"
#include "common.h"

namespace nt {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;
#ifndef NT_ATTN_WAVES
#define NT_ATTN_WAVES 8
#endif
constexpr int AW = NT_ATTN_WAVES;  // waves per workgroup
constexpr int SW = 32;             // cache slots per wave
constexpr int SWG = AW * SW;       // cache slots per workgroup (one split)
constexpr int QPAD = HD + 8;       // halves per staged query row
constexpr int OPAD = HD + 4;       // floats per staged output row
constexpr float PSCALE = 4096.f;   // p is split at 2^12 p
#ifndef NT_ATTN_MERGE_WAVES
#define NT_ATTN_MERGE_WAVES 4
#endif
constexpr int CWV = NT_ATTN_MERGE_WAVES;  // waves of the merge kernel
constexpr int CK = 16;             // splits per merge wave per round of loads

__device__ __forceinline__ h8 as_h8(u32x4 v) { return __builtin_bit_cast(h8, v); }

// The 32 slots of a wave starting at t0 (K rows, V groups of 8), loaded with the slots
// clamped into [0, n_ctx): a branch here would make the compiler wait for every load before
// the query staging.
struct KVTile {
  u32x4 k[2][4], v[8];
};
__device__ __forceinline__ void load_tile(KVTile& b, const uint16_t* kb, const uint16_t* vb, int t0, int n_ctx,
                                          int r, int qd) {
#pragma unroll
  for (int ta = 0; ta < 2; ++ta) {
    const int t = min(t0 + 8 * (r >> 2) + 4 * ta + (r & 3), n_ctx - 1);
    const uint8_t* p = reinterpret_cast<const uint8_t*>(kb + (size_t)t * HD + 8 * qd);
#pragma unroll
    for (int j = 0; j < 4; ++j) b.k[ta][j] = ld16(p + 64 * j);  // dims 32 j + 8 qd .. +7
  }
  const int grp = min((t0 >> 3) + qd, (n_ctx - 1) >> 3);
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(vb + ((size_t)grp * HD + r) * 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) b.v[j] = ld16(vp + 256 * j);  // dimension 16 j + r, slots 8 grp .. +7
}

template <int G>
__global__ __launch_bounds__(AW * 64) void attn_partial_kernel(const AttnArgs a) {
  constexpr int NB = (G + 7) / 8;  // column blocks of 8 heads (hi and lo columns each)
  constexpr int HPW = (G + AW - 1) / AW;  // query heads staged per wave
  __shared__ __attribute__((aligned(16))) _Float16 qx[NB][16][QPAD];
  __shared__ float qsig[NB * 8];
  __shared__ float ol[AW][NB][16][OPAD];
  __shared__ float wml[AW][NB * 8][2];

  const int split = blockIdx.x, g = blockIdx.y, tok = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, qd = lane >> 4;
  const int n_ctx = a.n_ctx + tok;
  const int n_split = (n_ctx + SWG - 1) / SWG;  // this token's splits
  if (split >= n_split) return;                  // the whole workgroup, before any barrier
  const float* qtok = a.q + (size_t)tok * a.q_stride;
  const int t0 = split * SWG + wave * SW;  // first slot of this wave

  // ---- 1. loads: this wave's query heads first (needed first), then its K and V tiles
  float2 qv[HPW];
#pragma unroll
  for (int k = 0; k < HPW; ++k) {  // unconditional (a wave past the group rereads its last head)
    const int hh = min(wave + AW * k, G - 1);
    qv[k] = *reinterpret_cast<const float2*>(qtok + (size_t)(g * G + hh) * HD + 2 * lane);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the query loads ahead of the cache loads
  const uint16_t* kb = a.k_cache + (size_t)g * a.max_ctx * HD;
  const uint16_t* vb = a.v_cache + (size_t)g * a.max_ctx * HD;
  KVTile cur;
  load_tile(cur, kb, vb, t0, n_ctx, r, qd);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. stage hi/lo fp16 parts of the scaled queries (columns of absent heads are zero)
  if (G < 8) {
    for (int i = threadIdx.x; i < 16 * QPAD; i += AW * 64)
      if (((i / QPAD) & 7) >= G) qx[0][i / QPAD][i % QPAD] = (_Float16)0.f;
  }
  if (threadIdx.x < NB * 8 && (int)threadIdx.x >= G) qsig[threadIdx.x] = 1.f;
  const float qscale = 1.4426950408889634f * 0.08838834764831845f;  // log2(e) / sqrt(128)
#pragma unroll
  for (int k = 0; k < HPW; ++k) {
    const int hh = wave + AW * k;
    if (hh < G) {
      float x0 = qv[k].x * qscale, x1 = qv[k].y * qscale;
      const float am = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      float sig = 1.f;
      if (am > 0.f) {
        int e;
        (void)frexpf(am, &e);
        sig = ldexpf(1.f, e - 14);  // am / sig in [2^13, 2^14)
      }
      const float inv = 1.f / sig;  // a power of two: exact
      x0 *= inv;
      x1 *= inv;
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      const int cb = hh >> 3, c = hh & 7;
      qx[cb][c][2 * lane] = h0;
      qx[cb][c][2 * lane + 1] = h1;
      qx[cb][c + 8][2 * lane] = (_Float16)(x0 - (float)h0);
      qx[cb][c + 8][2 * lane + 1] = (_Float16)(x1 - (float)h1);
      if (lane == 0) qsig[hh] = sig;
    }
  }
  __syncthreads();

  // B operand of lane (column r, quarter qd) for MFMA j = dims 32 j + 8 qd .. +7; each head's scale
  h8 bq[NB][4];
  float sig[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) bq[cb][j] = *reinterpret_cast<const h8*>(&qx[cb][r][32 * j + 8 * qd]);
    sig[cb] = qsig[cb * 8 + (r & 7)];
  }
  float mw[NB], lw[NB];  // the wave's maximum and sum for the lane's head (r & 7)
  f4 ow[NB][8];          // P V: rows 4 qd .. +3 (head rows, hi and lo), column r of dims 16 j ..
  if (t0 < n_ctx) {  // wave-uniform
    // ---- 3. scores: s[cb][k]: slot t0 + 8 qd + k, head 8 cb + (r & 7)
    float s[NB][8];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
      for (int ta = 0; ta < 2; ++ta) {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(cur.k[ta][j]), bq[cb][j], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = acc[i];
          v += dpp_mov<0x128>(v);  // row_ror:8 -> the head's other column (hi + lo)
          const int t = t0 + 8 * qd + 4 * ta + i;
          s[cb][4 * ta + i] = (t < n_ctx) ? v * sig[cb] : -INFINITY;
        }
      }
    }

    // V entries of slots past n_ctx may hold anything: zero them (0 * NaN would poison)
    if (t0 + SW > n_ctx) {
      const int nl = n_ctx - (t0 + 8 * qd);  // live slots of this lane's group of 8
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w4[4] = {cur.v[j].x, cur.v[j].y, cur.v[j].z, cur.v[j].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t keep = (2 * c + 1 < nl) ? 0xFFFFFFFFu : (2 * c < nl) ? 0x0000FFFFu : 0u;
          w4[c] &= keep;
        }
        cur.v[j] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }

    // ---- 4. softmax pieces over the wave's 32 slots, then P V
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      float m = s[cb][0];
#pragma unroll
      for (int k = 1; k < 8; ++k) m = fmaxf(m, s[cb][k]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));  // slot t0 is live: m is finite
      float l = 0.f;
      h8 pa;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = (s[cb][k] == -INFINITY) ? 0.f : exp2f(s[cb][k] - m);
        l += p;
        const float pp = p * PSCALE;
        const _Float16 hi = (_Float16)pp;
        pa[k] = (r < 8) ? hi : (_Float16)(pp - (float)hi);
      }
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      mw[cb] = m;
      lw[cb] = l;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        ow[cb][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, as_h8(cur.v[j]), f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
  }
  // the wave's part for the merge, written after all its products
  __builtin_amdgcn_sched_barrier(0);
  if (t0 < n_ctx) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      if (qd == 0 && r < 8) {
        wml[wave][cb * 8 + r][0] = mw[cb];
        wml[wave][cb * 8 + r][1] = lw[cb];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ol[wave][cb][4 * qd + i][16 * j + r] = ow[cb][j][i];
    }
  } else if (lane < NB * 8) {
    wml[wave][lane][0] = -INFINITY;
    wml[wave][lane][1] = 0.f;
  }
  __syncthreads();

  // ---- 5. merge the waves (rows h and h + 8 of a column block are one head's hi and lo)
  for (int idx = threadIdx.x; idx < G * HD; idx += AW * 64) {
    const int h = idx >> 7, d = idx & (HD - 1);
    const int cb = h >> 3, hr = h & 7;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < AW; ++w) M = fmaxf(M, wml[w][h][0]);
    float v = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < AW; ++w) {
      const float mw = wml[w][h][0];
      if (mw != -INFINITY) {
        const float f = exp2f(mw - M);
        v += (ol[w][cb][hr][d] + ol[w][cb][hr + 8][d]) * f;
        L += wml[w][h][1] * f;
      }
    }
    v *= 1.f / PSCALE;
    if (n_split == 1) {
      a.out[(size_t)tok * a.out_stride + (size_t)(g * G + h) * HD + d] = v / L;
    } else {
      float* po = a.part + (size_t)tok * a.part_stride + (((size_t)g * n_split + split) * G + h) * (HD + 2);
      po[d] = v;
      if (d == 0) {
        po[HD] = M;
        po[HD + 1] = L;
      }
    }
  }
}

// Merge of the splits' partials: one workgroup per query head.  Wave w takes splits
// w, w + 4, ...; lane = output dimensions 2 lane, 2 lane + 1.  Every split's maximum
// and sum go through LDS; the output loads of the first 64 splits are issued together
// with them.
template <int G>
__global__ __launch_bounds__(CWV * 64) void attn_combine_kernel(const AttnArgs a) {
  extern __shared__ float cm[];  // [n_split] maxima, then [n_split] sums
  __shared__ float red[CWV][HD];
  __shared__ float wred[CWV][2];
  const int hq = blockIdx.x, tok = blockIdx.y;
  const int g = hq / G, hg = hq % G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ns = (a.n_ctx + tok + SWG - 1) / SWG;  // this token's splits
  if (ns == 1) return;  // the partial kernel wrote this token's output itself
  const float* gp = a.part + (size_t)tok * a.part_stride + ((size_t)g * ns * G + hg) * (HD + 2);
  const size_t ss = (size_t)G * (HD + 2);

  float2 ov[CK];
#pragma unroll
  for (int k = 0; k < CK; ++k) {
    const int sp = wave + CWV * k;
    if (sp < ns) ov[k] = *reinterpret_cast<const float2*>(gp + sp * ss + 2 * lane);
  }
  float mloc = -INFINITY;
  for (int sp = threadIdx.x; sp < ns; sp += CWV * 64) {
    const float m = gp[sp * ss + HD];
    cm[sp] = m;
    cm[ns + sp] = gp[sp * ss + HD + 1];
    mloc = fmaxf(mloc, m);
  }
  mloc = wave_max(mloc);
  if (lane == 0) wred[wave][0] = mloc;
  __syncthreads();
  float M = wred[0][0];
#pragma unroll
  for (int w = 1; w < CWV; ++w) M = fmaxf(M, wred[w][0]);
  float lloc = 0.f;
  for (int sp = threadIdx.x; sp < ns; sp += CWV * 64) lloc += cm[ns + sp] * exp2f(cm[sp] - M);
  lloc = wave_sum(lloc);
  if (lane == 0) wred[wave][1] = lloc;

  float o0 = 0.f, o1 = 0.f;
  for (int base = 0;; base += CWV * CK) {
#pragma unroll
    for (int k = 0; k < CK; ++k) {
      const int sp = base + wave + CWV * k;
      if (sp < ns) {
        const float f = exp2f(cm[sp] - M);
        o0 += ov[k].x * f;
        o1 += ov[k].y * f;
      }
    }
    if (base + CWV * CK >= ns) break;
#pragma unroll
    for (int k = 0; k < CK; ++k) {
      const int sp = base + CWV * CK + wave + CWV * k;
      if (sp < ns) ov[k] = *reinterpret_cast<const float2*>(gp + sp * ss + 2 * lane);
    }
  }
  red[wave][2 * lane] = o0;
  red[wave][2 * lane + 1] = o1;
  __syncthreads();
  if (threadIdx.x < HD) {
    float L = 0.f, v = 0.f;
#pragma unroll
    for (int w = 0; w < CWV; ++w) {
      L += wred[w][1];
      v += red[w][threadIdx.x];
    }
    a.out[(size_t)tok * a.out_stride + (size_t)hq * HD + threadIdx.x] = v / L;
  }
}

int attn_n_split(int n_ctx) { return (n_ctx + SWG - 1) / SWG; }

static int attn_max_split() { return ATTN_MAX_CTX / SWG; }

size_t attn_part_floats(int n_q, int max_ctx) {
  return (size_t)attn_n_split(max_ctx) * (size_t)n_q * (HD + 2);
}

template <int G>
static hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_partial_kernel<G>, dim3(a.n_split, a.n_kv, a.n_tok), dim3(AW * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;  // then every token has one split
  hipLaunchKernelGGL(attn_combine_kernel<G>, dim3(a.n_kv * G, a.n_tok), dim3(CWV * 64), 2 * sizeof(float) * a.n_split,
                     s, a);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnArgs& a, int group, hipStream_t s) {
  if (a.n_tok < 1 || a.n_split != attn_n_split(a.n_ctx + a.n_tok - 1) || a.n_split > attn_max_split() ||
      a.max_ctx % 8 || a.n_ctx + a.n_tok - 1 > a.max_ctx)
    return hipErrorInvalidValue;
  if (a.n_tok > 1 && (a.q_stride < (int64_t)a.n_kv * group * HD || a.out_stride < (int64_t)a.n_kv * group * HD ||
                      a.part_stride < (int64_t)attn_part_floats(a.n_kv * group, a.n_ctx + a.n_tok - 1)))
    return hipErrorInvalidValue;
  switch (group) {
    case 1: return launch_g<1>(a, s);
    case 2: return launch_g<2>(a, s);
    case 4: return launch_g<4>(a, s);
    case 8: return launch_g<8>(a, s);
    case 16: return launch_g<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nt
