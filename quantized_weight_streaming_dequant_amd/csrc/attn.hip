// GQA decode attention over an fp16 KV cache, one new token, gfx950.
//
// The pages' layer has GQA attention over a KV cache kept in fp16 (ntransformer
// overview, de.news.hada.io, "Hauptfunktionen" and "Roadmap der
// Entwicklungsphasen"), with a softmax kernel ("Architektur und Codestruktur").
// With only 8 KV heads, one workgroup per head would leave most of the chip idle,
// so the cache is split along the sequence: workgroup (split, kv head) handles a
// run of slots for all query heads of the group (K and V rows are read once per
// group), each of its four waves a quarter of the run.  A wave keeps the group's
// scores in registers (one slot per lane), takes the max-subtracted exponentials
// with exp2, and accumulates p * V with lanes over the 128 dimensions.  Waves merge
// through LDS; workgroups write (max, sum, unnormalised output) partials, and the
// last workgroup of each KV head to finish (an atomic counter in the workspace,
// reset by that workgroup) merges the splits.
#include "attn.h"
#include "common.h"

namespace nt {

constexpr int HD = 128;
constexpr int AW = 4;  // waves per workgroup

template <int G>
__global__ __launch_bounds__(AW * 64) void attn_decode_kernel(const AttnArgs a) {
  __shared__ float4 qs4[G * HD / 4];
  __shared__ float pe[AW][G][64];
  __shared__ float wpart[AW][G][HD + 2];
  __shared__ int last_flag;
  float* qs = reinterpret_cast<float*>(qs4);

  const int split = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int cw = a.slots_per_wave;
  const int t0 = split * (AW * cw) + wave * cw;  // first slot of this wave

  // q of the group's heads, scaled by log2(e)/sqrt(HD) so that scores are in exp2 units
  const float qscale = 1.4426950408889634f * 0.08838834764831845f;
  for (int i = threadIdx.x; i < G * HD; i += AW * 64) qs[i] = a.q[(size_t)(g * G) * HD + i] * qscale;
  __syncthreads();

  // scores: lane = one slot
  const int t = t0 + lane;
  const bool live = lane < cw && t < a.n_ctx;
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  if (live) {
    const uint8_t* kr = reinterpret_cast<const uint8_t*>(a.k_cache + ((size_t)g * a.max_ctx + t) * HD);
#pragma unroll 4
    for (int c = 0; c < HD / 8; ++c) {
      const u32x4 kv = ld16(kr + 16 * c);
      const uint32_t w4[4] = {kv.x, kv.y, kv.z, kv.w};
      float kf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kf[2 * j] = h2f(w4[j]);
        kf[2 * j + 1] = h2f(w4[j] >> 16);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 qa = qs4[(h * HD + 8 * c) / 4];
        const float4 qb = qs4[(h * HD + 8 * c) / 4 + 1];
        s[h] += qa.x * kf[0] + qa.y * kf[1] + qa.z * kf[2] + qa.w * kf[3] + qb.x * kf[4] + qb.y * kf[5] +
                qb.z * kf[6] + qb.w * kf[7];
      }
    }
  }
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = wave_max(live ? s[h] : -INFINITY);
    const float e = live ? exp2f(s[h] - m[h]) : 0.f;  // m is -inf only if no slot is live
    l[h] = wave_sum(e);
    pe[wave][h][lane] = e;
  }
  __syncthreads();

  // p V: lane = dimensions 2 lane, 2 lane + 1
  float o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) o0[h] = o1[h] = 0.f;
  const int nt = min(cw, a.n_ctx - t0);
  const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.v_cache + ((size_t)g * a.max_ctx + t0) * HD + 2 * lane);
#pragma unroll 4
  for (int j = 0; j < nt; ++j) {
    const uint32_t vv = ld4(vb + (size_t)j * HD * 2);
    const float v0 = h2f(vv), v1 = h2f(vv >> 16);
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

  // merge the four waves: partial of this split, written to the workspace
  float* part = a.part + (((size_t)g * a.n_split + split) * G) * (HD + 2);
  for (int i = threadIdx.x; i < G * (HD + 2); i += AW * 64) {
    const int h = i / (HD + 2), d = i % (HD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < AW; ++w) M = fmaxf(M, wpart[w][h][HD]);
    float v = 0.f;
    if (M != -INFINITY) {
      if (d == HD) {
        v = M;
      } else {
#pragma unroll
        for (int w = 0; w < AW; ++w) {
          const float mw = wpart[w][h][HD];
          if (mw != -INFINITY) v += wpart[w][h][d] * exp2f(mw - M);
        }
      }
    } else if (d == HD) {
      v = -INFINITY;
    }
    part[i] = v;
  }

  // last workgroup of this KV head merges all splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(a.counter + g, 1);
    last_flag = (prev == a.n_split - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  const float* gp = a.part + ((size_t)g * a.n_split * G) * (HD + 2);
  for (int i = threadIdx.x; i < G * (HD / 2); i += AW * 64) {
    const int h = i / (HD / 2), d = 2 * (i % (HD / 2));
    float M = -INFINITY;
    for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, __builtin_nontemporal_load(gp + ((size_t)sp * G + h) * (HD + 2) + HD));
    float L = 0.f, r0 = 0.f, r1 = 0.f;
    for (int sp = 0; sp < a.n_split; ++sp) {
      const float* pp = gp + ((size_t)sp * G + h) * (HD + 2);
      const float ms = __builtin_nontemporal_load(pp + HD);
      if (ms == -INFINITY) continue;
      const float f = exp2f(ms - M);
      L += __builtin_nontemporal_load(pp + HD + 1) * f;
      r0 += __builtin_nontemporal_load(pp + d) * f;
      r1 += __builtin_nontemporal_load(pp + d + 1) * f;
    }
    const float inv = 1.0f / L;
    a.out[((size_t)(g * G + h)) * HD + d] = r0 * inv;
    a.out[((size_t)(g * G + h)) * HD + d + 1] = r1 * inv;
  }
  if (threadIdx.x == 0) atomicExch(a.counter + g, 0);
}

int attn_slots_per_wave(int n_ctx, int n_kv) {
  // enough workgroups to cover the chip: aim for >= 256 (split, head) pairs
  for (int cw = 16; cw <= 64; cw *= 2) {
    const int n_split = (n_ctx + AW * cw - 1) / (AW * cw);
    if (n_split * n_kv <= 512) return cw;
  }
  return 64;
}

int attn_n_split(int n_ctx, int slots_per_wave) { return (n_ctx + AW * slots_per_wave - 1) / (AW * slots_per_wave); }

size_t attn_part_floats(int n_q, int max_ctx) {
  const int max_split = (max_ctx + AW * 16 - 1) / (AW * 16);
  return (size_t)max_split * (size_t)n_q * (HD + 2);
}

hipError_t attn_launch(const AttnArgs& a, int group, hipStream_t s) {
  const dim3 grid(a.n_split, a.n_kv), block(AW * 64);
  switch (group) {
    case 1: hipLaunchKernelGGL(attn_decode_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(attn_decode_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_decode_kernel<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(attn_decode_kernel<8>, grid, block, 0, s, a); break;
    case 16: hipLaunchKernelGGL(attn_decode_kernel<16>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nt
