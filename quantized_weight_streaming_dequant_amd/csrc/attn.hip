// GQA decode attention over an fp16 KV cache, one new token, gfx950.
//
// The pages' layer has GQA attention over a KV cache kept in fp16 (ntransformer
// overview, de.news.hada.io, "Hauptfunktionen" and "Roadmap der
// Entwicklungsphasen"), with a softmax kernel ("Architektur und Codestruktur").
// With only 8 KV heads, one workgroup per head would leave most of the chip idle, so
// the cache is split along the sequence: workgroup (split, kv head) handles a run of
// 4*cw slots for all query heads of the group (each K and V row is read once per
// group), each of its four waves cw of them.  The kernel is bound by load latency, so
// every lane issues all of its K and V loads before it computes anything:
//  * scores: 64/cw lanes per slot, each over its share of the 128 dimensions (K rows
//    read as contiguous 16-byte pieces), combined with lane shuffles;
//  * max-subtracted exponentials in exp2 units (q is pre-scaled by log2(e)/sqrt(128));
//  * p V: lane = two of the 128 output dimensions, one 4-byte V load per slot;
//  * the four waves merge through LDS into one (max, sum, unnormalised output) partial
//    per head, written to the workspace;
//  * a second kernel, one workgroup per query head, merges the splits' partials.
#include "attn.h"
#include "common.h"

namespace nt {

constexpr int HD = 128;
constexpr int AW = 4;          // waves per workgroup
constexpr int MAX_SPLIT_FAST = 32;  // splits merged with one round of loads

template <int G, int CW>
__global__ __launch_bounds__(AW * 64) void attn_decode_kernel(const AttnArgs a) {
  constexpr int LPS = 64 / CW;    // lanes per slot in the score phase
  constexpr int DPL = HD / LPS;   // dimensions per lane in the score phase
  __shared__ float4 qs4[G * HD / 4];
  __shared__ float pe[AW][G][CW];
  __shared__ float wpart[AW][G][HD + 2];
  float* qs = reinterpret_cast<float*>(qs4);

  const int split = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = split * (AW * CW) + wave * CW;  // first slot of this wave

  // ---- issue every global load of this wave first
  const int slot = lane / LPS, part = lane % LPS;
  const int t = t0 + slot;
  const bool live = t < a.n_ctx;
  u32x4 kv[DPL / 8];
  {
    const uint8_t* kr = reinterpret_cast<const uint8_t*>(a.k_cache + ((size_t)g * a.max_ctx + (live ? t : 0)) * HD +
                                                         part * DPL);
#pragma unroll
    for (int c = 0; c < DPL / 8; ++c) kv[c] = live ? ld16(kr + 16 * c) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t vv[CW];
  {
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v_cache + ((size_t)g * a.max_ctx) * HD + 2 * lane);
#pragma unroll
    for (int j = 0; j < CW; ++j) vv[j] = (t0 + j < a.n_ctx) ? ld4(vb + (size_t)(t0 + j) * HD * 2) : 0u;
  }
  // q of the group's heads, scaled so that scores come out in exp2 units
  const float qscale = 1.4426950408889634f * 0.08838834764831845f;
  for (int i = threadIdx.x; i < G * HD; i += AW * 64) qs[i] = a.q[(size_t)(g * G) * HD + i] * qscale;
  __syncthreads();

  // ---- scores over this lane's dimensions, combined across the slot's lanes
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
  for (int c = 0; c < DPL / 8; ++c) {
    const uint32_t w4[4] = {kv[c].x, kv[c].y, kv[c].z, kv[c].w};
    float kf[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kf[2 * j] = h2f(w4[j]);
      kf[2 * j + 1] = h2f(w4[j] >> 16);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4 qa = qs4[(h * HD + part * DPL + 8 * c) / 4];
      const float4 qb = qs4[(h * HD + part * DPL + 8 * c) / 4 + 1];
      s[h] += qa.x * kf[0];
      s[h] += qa.y * kf[1];
      s[h] += qa.z * kf[2];
      s[h] += qa.w * kf[3];
      s[h] += qb.x * kf[4];
      s[h] += qb.y * kf[5];
      s[h] += qb.z * kf[6];
      s[h] += qb.w * kf[7];
    }
  }
#pragma unroll
  for (int off = 1; off < LPS; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] += __shfl_xor(s[h], off, 64);
  }

  // ---- softmax pieces of this wave
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = wave_max(live ? s[h] : -INFINITY);
    const float e = live ? exp2f(s[h] - m[h]) : 0.f;  // m is -inf only if no slot is live
    l[h] = wave_sum(part == 0 ? e : 0.f);
    if (part == 0) pe[wave][h][slot] = e;
  }
  __syncthreads();

  // ---- p V: lane = dimensions 2 lane, 2 lane + 1
  float o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) o0[h] = o1[h] = 0.f;
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const float v0 = h2f(vv[j]), v1 = h2f(vv[j] >> 16);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = pe[wave][h][j];
      o0[h] += p * v0;
      o1[h] += p * v1;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    wpart[wave][h][2 * lane] = o0[h];
    wpart[wave][h][2 * lane + 1] = o1[h];
    if (lane == 0) {
      wpart[wave][h][HD] = m[h];
      wpart[wave][h][HD + 1] = l[h];
    }
  }
  __syncthreads();

  // ---- merge the four waves: this split's partial, written to the workspace
  float* part_out = a.part + (((size_t)g * a.n_split + split) * G) * (HD + 2);
  for (int i = threadIdx.x; i < G * (HD + 2); i += AW * 64) {
    const int h = i / (HD + 2), d = i % (HD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < AW; ++w) M = fmaxf(M, wpart[w][h][HD]);
    float v;
    if (d == HD) {
      v = M;
    } else if (M == -INFINITY) {
      v = 0.f;
    } else {
      v = 0.f;
#pragma unroll
      for (int w = 0; w < AW; ++w) {
        const float mwv = wpart[w][h][HD];
        if (mwv != -INFINITY) v += wpart[w][h][d] * exp2f(mwv - M);
      }
    }
    part_out[i] = v;
  }
}

// Merge of the splits' partials: one workgroup per query head, lane = two output
// dimensions; every partial of the head is loaded in one round per 32 splits.
template <int G>
__global__ __launch_bounds__(64) void attn_combine_kernel(const AttnArgs a) {
  __shared__ float ms[MAX_SPLIT_FAST], ls[MAX_SPLIT_FAST];
  const int hq = blockIdx.x;  // query head
  const int g = hq / G, hg = hq % G;
  const int lane = threadIdx.x;
  const int d = 2 * lane;
  const float* gp = a.part + ((size_t)g * a.n_split * G + hg) * (HD + 2);  // split sp at gp + sp*G*(HD+2)
  const size_t sstride = (size_t)G * (HD + 2);
  float runM = -INFINITY, runL = 0.f, r0 = 0.f, r1 = 0.f;
  for (int base = 0; base < a.n_split; base += MAX_SPLIT_FAST) {
    const int nb = min(MAX_SPLIT_FAST, a.n_split - base);
    if (lane < nb) {
      ms[lane] = gp[(size_t)(base + lane) * sstride + HD];
      ls[lane] = gp[(size_t)(base + lane) * sstride + HD + 1];
    }
    float2 ov[MAX_SPLIT_FAST];
#pragma unroll
    for (int k = 0; k < MAX_SPLIT_FAST; ++k)
      if (k < nb) ov[k] = *reinterpret_cast<const float2*>(gp + (size_t)(base + k) * sstride + d);
    __syncthreads();
    float M = runM;
#pragma unroll
    for (int k = 0; k < MAX_SPLIT_FAST; ++k)
      if (k < nb) M = fmaxf(M, ms[k]);
    const float f0 = (runM == -INFINITY) ? 0.f : exp2f(runM - M);
    runL *= f0;
    r0 *= f0;
    r1 *= f0;
#pragma unroll
    for (int k = 0; k < MAX_SPLIT_FAST; ++k) {
      if (k < nb && ms[k] != -INFINITY) {
        const float f = exp2f(ms[k] - M);
        runL += ls[k] * f;
        r0 += ov[k].x * f;
        r1 += ov[k].y * f;
      }
    }
    runM = M;
    __syncthreads();  // ms/ls are rewritten by the next chunk
  }
  const float inv = 1.0f / runL;
  *reinterpret_cast<float2*>(a.out + (size_t)hq * HD + d) = make_float2(r0 * inv, r1 * inv);
}

int attn_slots_per_wave(int n_ctx, int n_kv) {
  (void)n_kv;
  // the smallest run per wave that keeps the merge within two rounds of loads
  for (int cw = 16; cw < 64; cw *= 2)
    if ((n_ctx + AW * cw - 1) / (AW * cw) <= 2 * MAX_SPLIT_FAST) return cw;
  return 64;
}

int attn_n_split(int n_ctx, int slots_per_wave) { return (n_ctx + AW * slots_per_wave - 1) / (AW * slots_per_wave); }

size_t attn_part_floats(int n_q, int max_ctx) {
  const int max_split = (max_ctx + AW * 16 - 1) / (AW * 16);
  return (size_t)max_split * (size_t)n_q * (HD + 2);
}

template <int G>
static hipError_t launch_g(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_split, a.n_kv), block(AW * 64);
  switch (a.slots_per_wave) {
    case 16: hipLaunchKernelGGL((attn_decode_kernel<G, 16>), grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL((attn_decode_kernel<G, 32>), grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL((attn_decode_kernel<G, 64>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel<G>, dim3(a.n_kv * G), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t attn_launch(const AttnArgs& a, int group, hipStream_t s) {
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
