// Decode-layer pieces for several tokens at consecutive positions, other than the GEMMs and
// the attention: the verification pass of self-speculative decoding runs a layer over the
// k draft tokens at once (ntransformer overview, de.news.hada.io, "Hauptfunktionen":
// self-speculative decoding; RMSNorm, RoPE and the KV cache of the Llama layer).  These
// move a few hundred KB per layer and are latency-bound: one workgroup per token row.
#include "common.h"
#include "layer_k.h"

namespace nt {

// one workgroup of 1024 threads per row: each thread holds up to RN_V float4 of its row in
// registers, so x is read once, with all of a thread's loads in flight together
constexpr int RN_T = 1024;
constexpr int RN_V = 8;  // rows up to RN_T * RN_V * 4 = 32768 floats

__global__ __launch_bounds__(RN_T) void rmsnorm_rows_kernel(int n, const float* __restrict__ x,
                                                            const float* __restrict__ g, float eps,
                                                            float* __restrict__ y, float* __restrict__ copy) {
  __shared__ float red[RN_T / 64];
  const size_t row = (size_t)blockIdx.x * n;
  const float4* xr = reinterpret_cast<const float4*>(x + row);
  const int n4 = n >> 2;
  float4 v[RN_V];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < RN_V; ++j) {
    const int i = (int)threadIdx.x + j * RN_T;
    v[j] = i < n4 ? xr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int j = 0; j < RN_V; ++j) ss += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < RN_T / 64; ++w) tot += red[w];
  const float scale = 1.0f / sqrtf(tot / (float)n + eps);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4* y4 = reinterpret_cast<float4*>(y + row);
  float4* c4 = copy ? reinterpret_cast<float4*>(copy + row) : nullptr;
#pragma unroll
  for (int j = 0; j < RN_V; ++j) {
    const int i = (int)threadIdx.x + j * RN_T;
    if (i < n4) {
      const float4 gg = g4[i];
      y4[i] = make_float4(v[j].x * scale * gg.x, v[j].y * scale * gg.y, v[j].z * scale * gg.z, v[j].w * scale * gg.w);
      if (c4) c4[i] = v[j];
    }
  }
}

hipError_t rmsnorm_rows_launch(int n_rows, int n, const float* x, const float* gain, float eps, float* y, float* copy,
                               hipStream_t s) {
  if (n % 4 || n > RN_T * RN_V * 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(n_rows), dim3(RN_T), 0, s, n, x, gain, eps, y, copy);
  return hipGetLastError();
}

// workgroup (token t, head): thread i < 64 turns pair i of the head; for a KV head it also
// writes the fp16 k pair and the two v values of dimensions 2i, 2i + 1
__global__ __launch_bounds__(64) void rope_append_kernel(int n_q, int n_kv, int pos, double theta, float* __restrict__ q,
                                                         const float* __restrict__ k, const float* __restrict__ v,
                                                         uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                                                         int max_ctx) {
  constexpr int HD = 128;
  const int t = blockIdx.x, head = blockIdx.y, i = threadIdx.x;
  const int p = pos + t;
  const float2 c = rope_cs(theta, p, i, HD);
  if (head < n_q) {
    float* r = q + ((size_t)t * n_q + head) * HD + 2 * i;
    const float x0 = r[0], x1 = r[1];
    r[0] = x0 * c.x - x1 * c.y;
    r[1] = x0 * c.y + x1 * c.x;
  } else {
    const int g = head - n_q;
    const float* kr = k + ((size_t)t * n_kv + g) * HD + 2 * i;
    const float x0 = kr[0], x1 = kr[1];
    uint16_t* kp = kc + ((size_t)g * max_ctx + p) * HD + 2 * i;
    kp[0] = f2h_rne(x0 * c.x - x1 * c.y);
    kp[1] = f2h_rne(x0 * c.y + x1 * c.x);
    const float* vr = v + ((size_t)t * n_kv + g) * HD + 2 * i;
    uint16_t* vp = vc + (size_t)g * max_ctx * HD + ((size_t)(p >> 3) * HD + 2 * i) * 8 + (p & 7);
    vp[0] = f2h_rne(vr[0]);
    vp[8] = f2h_rne(vr[1]);
  }
}

hipError_t rope_append_launch(int n_tok, int n_q, int n_kv, int pos, double theta, float* q, const float* k,
                              const float* v, uint16_t* k_cache, uint16_t* v_cache, int max_ctx, hipStream_t s) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(n_tok, n_q + n_kv), dim3(64), 0, s, n_q, n_kv, pos, theta, q, k, v,
                     k_cache, v_cache, max_ctx);
  return hipGetLastError();
}

}  // namespace nt
