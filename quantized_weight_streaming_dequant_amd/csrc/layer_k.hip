// Decode-layer pieces for several tokens at consecutive positions, other than the GEMMs and
// the attention: the verification pass of self-speculative decoding runs a layer over the
// k draft tokens at once (ntransformer overview, de.news.hada.io, "Hauptfunktionen":
// self-speculative decoding; RMSNorm, RoPE and the KV cache of the Llama layer).  These
// move a few hundred KB per layer and are latency-bound: one workgroup per token row.
#include "common.h"
#include "layer_k.h"

namespace nt {

__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(int n, const float* __restrict__ x,
                                                           const float* __restrict__ g, float eps, float* __restrict__ y,
                                                           float* __restrict__ copy) {
  __shared__ float red[4];
  const size_t row = (size_t)blockIdx.x * n;
  const float* xr = x + row;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ss += xr[i] * xr[i];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float scale = 1.0f / sqrtf(tot / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float v = xr[i];
    y[row + i] = v * scale * g[i];
    if (copy) copy[row + i] = v;
  }
}

hipError_t rmsnorm_rows_launch(int n_rows, int n, const float* x, const float* gain, float eps, float* y, float* copy,
                               hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(n_rows), dim3(256), 0, s, n, x, gain, eps, y, copy);
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
