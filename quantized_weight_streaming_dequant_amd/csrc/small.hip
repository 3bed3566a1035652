// Stand-alone decode-path kernels: dequantize (test hook), RMSNorm, RoPE, SwiGLU,
// embedding row, argmax.  In the fused layer these steps run inside the GEMV
// prologues/epilogues (gemv.hip); the stand-alone forms serve the per-op C ABI.
// Ops from the ntransformer overview (de.news.hada.io), "Hauptfunktionen" and
// "Architektur und Codestruktur"; block formats from "Überblick über NTransformer".
#include "common.h"
#include "small.h"

namespace nt {

// ------------------------------------------------------------ dequantize
// One thread per 32 weights.  Every product below is exact in fp32 (at most 24
// significant bits), so the single rounding happens at the Q4_K subtraction and the
// result is the exact weight rounded once to fp32.

__device__ __forceinline__ uint32_t byte_at(const uint8_t* p, int i) { return p[i]; }
__device__ __forceinline__ float f16_at(const uint8_t* p) { return h2f((uint32_t)p[0] | ((uint32_t)p[1] << 8)); }

__device__ void dequant_group(int fmt, const uint8_t* blk, int grp, float* out) {
  if (fmt == FMT_F16) {  // 32 consecutive binary16 weights at blk
    for (int i = 0; i < 32; ++i) out[i] = f16_at(blk + 2 * i);
  } else if (fmt == FMT_F32) {
    for (int i = 0; i < 32; ++i) out[i] = *reinterpret_cast<const float*>(blk + 4 * i);
  } else if (fmt == FMT_Q8_0) {
    const float d = f16_at(blk);
    for (int i = 0; i < 32; ++i) out[i] = d * (float)(int8_t)blk[2 + i];
  } else if (fmt == FMT_Q4_0) {
    const float d = f16_at(blk);
    for (int i = 0; i < 32; ++i) {
      const int n = i < 16 ? (blk[2 + i] & 15) : (blk[2 + i - 16] >> 4);
      out[i] = d * (float)(n - 8);
    }
  } else if (fmt == FMT_Q4_K || fmt == FMT_Q5_K) {
    // grp = sub-block j (32 weights); Q5_K adds bit j of high byte l, worth 16
    const int j = grp;
    const float d = f16_at(blk), dmin = f16_at(blk + 2);
    const uint8_t* S = blk + 4;
    int sc, m;
    if (j < 4) {
      sc = S[j] & 63;
      m = S[j + 4] & 63;
    } else {
      sc = (S[j + 4] & 15) | ((S[j - 4] >> 6) << 4);
      m = (S[j + 4] >> 4) | ((S[j] >> 6) << 4);
    }
    const float dsc = d * (float)sc, dm = dmin * (float)m;
    const bool k5 = fmt == FMT_Q5_K;
    const uint8_t* Q = blk + (k5 ? 48 : 16) + 32 * (j >> 1);
    const uint8_t* H = blk + 16;
    const int shift = 4 * (j & 1);
    for (int l = 0; l < 32; ++l) {
      const int q = ((Q[l] >> shift) & 15) + (k5 ? 16 * ((H[l] >> j) & 1) : 0);
      out[l] = dsc * (float)q - dm;
    }
  } else {
    // Q6_K, grp = 32-weight run: h = grp/4, t = grp%4
    const int h = grp >> 2, t = grp & 3;
    const uint8_t* QL = blk + 64 * h + 32 * (t & 1);
    const uint8_t* QH = blk + 128 + 32 * h;
    const int8_t* sc = reinterpret_cast<const int8_t*>(blk + 192);
    const float d = f16_at(blk + 208);
    for (int l = 0; l < 32; ++l) {
      const int q = ((QL[l] >> (4 * (t >> 1))) & 15) | (((QH[l] >> (2 * t)) & 3) << 4);
      const float ds = d * (float)sc[8 * h + 2 * t + (l >> 4)];
      out[l] = ds * (float)(q - 32);
    }
  }
}

// Superblock b of a Q4_KT row (tiles of 16, common.h) gathered back into Q4_K's byte order.
__device__ void q4kt_gather(const uint8_t* row, int nsb, int b, uint8_t* out) {
  const uint8_t* hd = row + q4kt_head(nsb, b);
  for (int i = 0; i < 16; ++i) out[i] = hd[i];
  for (int g = 0; g < 4; ++g) {
    const uint8_t* qa = row + q4kt_qa(nsb, b, g);
    const uint8_t* qb = row + q4kt_qb(nsb, b, g);
    for (int i = 0; i < 16; ++i) {
      out[16 + 32 * g + i] = qa[i];
      out[32 + 32 * g + i] = qb[i];
    }
  }
}

// 32 weights of group grp (of block b) of a row starting at row, any format.
__device__ void dequant_row_group(int fmt, const uint8_t* row, int64_t cols, int64_t b, int grp, float* out) {
  if (fmt == FMT_Q4_KT) {
    uint8_t blk[144];
    q4kt_gather(row, (int)(cols >> 8), (int)b, blk);
    dequant_group(FMT_Q4_K, blk, grp, out);
  } else if (fmt == FMT_Q5_KT) {  // superblock b of a Q5_KT row gathered back into Q5_K's byte order
    const int nsb = (int)(cols >> 8);
    uint8_t blk[176];
    for (int i = 0; i < 16; ++i) {
      blk[i] = row[q5kt_hd(nsb, (int)b) + i];
      blk[16 + i] = row[q5kt_ha(nsb, (int)b) + i];
      blk[32 + i] = row[q5kt_hb(nsb, (int)b) + i];
    }
    for (int g = 0; g < 4; ++g)
      for (int i = 0; i < 16; ++i) {
        blk[48 + 32 * g + i] = row[q5kt_qa(nsb, (int)b, g) + i];
        blk[64 + 32 * g + i] = row[q5kt_qb(nsb, (int)b, g) + i];
      }
    dequant_group(FMT_Q5_K, blk, grp, out);
  } else if (fmt == FMT_Q8_0T) {  // block b of a Q8_0T row gathered back into Q8_0's byte order
    const int nb = (int)(cols >> 5);
    uint8_t blk[34];
    for (int i = 0; i < 2; ++i) blk[i] = row[q8t_d(nb, (int)b) + i];
    for (int i = 0; i < 16; ++i) {
      blk[2 + i] = row[q8t_qa(nb, (int)b) + i];
      blk[18 + i] = row[q8t_qb(nb, (int)b) + i];
    }
    dequant_group(FMT_Q8_0, blk, grp, out);
  } else {
    dequant_group(fmt, row + b * block_bytes(fmt), grp, out);
  }
}

__global__ void dequant_kernel(int fmt, int64_t rows, int64_t cols, const uint8_t* __restrict__ blocks,
                               float* __restrict__ w) {
  const int be = block_elems(fmt), bb = block_bytes(fmt);
  const int64_t groups_per_row = cols / 32;
  const int64_t total = rows * groups_per_row;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < total; gi += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = gi / groups_per_row, cg = gi % groups_per_row;
    const int64_t c0 = cg * 32;
    const int64_t b = c0 / be;
    const int grp = (int)((c0 % be) / 32);
    float tmp[32];
    dequant_row_group(fmt, blocks + r * (cols / be) * bb, cols, b, grp, tmp);
    float* o = w + r * cols + c0;
    for (int i = 0; i < 32; ++i) o[i] = tmp[i];
  }
}

// Q4_K -> Q4_KT: one thread per 16-byte part of the output.  Part k of tile t (m superblocks)
// is, in the tile's Q4_K bytes (9 parts per superblock: header, then code bytes in 16-byte
// runs), part 9k (k < m: headers), 9j + 1 + 2g (k = m + 4j + g: first halves of the quarters)
// or 9j + 2 + 2g (k = 5m + 4j + g: second halves).
__global__ void repack_q4kt_kernel(int64_t rows, int nsb, const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  const int64_t per_row = 9 * (int64_t)nsb, total = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row;
    const int c = (int)(i % per_row);
    const int t = c / 144, k = c % 144;
    const int m = nsb - 16 * t < 16 ? nsb - 16 * t : 16;
    int from;
    if (k < m) from = 9 * k;
    else if (k < 5 * m) from = 9 * ((k - m) >> 2) + 1 + 2 * ((k - m) & 3);
    else from = 9 * ((k - 5 * m) >> 2) + 2 + 2 * ((k - 5 * m) & 3);
    const int64_t tile = r * 144 * (int64_t)nsb + 2304 * (int64_t)t;
    *reinterpret_cast<uint4*>(dst + tile + 16 * k) = *reinterpret_cast<const uint4*>(src + tile + 16 * from);
  }
}

hipError_t repack_q4kt_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s) {
  const int64_t total = rows * 9 * (cols >> 8);
  const int64_t nb = (total + 255) / 256;
  const int grid = (int)(nb < 65536 ? nb : 65536);
  hipLaunchKernelGGL(repack_q4kt_kernel, dim3(grid), dim3(256), 0, s, rows, (int)(cols >> 8),
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<uint8_t*>(dst));
  return hipGetLastError();
}

// Q8_0 -> Q8_0T: one thread per block, its 34 bytes (at a 2-byte phase) moved as bytes.
__global__ void repack_q8t_kernel(int64_t rows, int nb, const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  const int64_t total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb;
    const int b = (int)(i % nb);
    const uint8_t* in = src + r * 34 * (int64_t)nb + 34 * (int64_t)b;
    uint8_t* row = dst + r * 34 * (int64_t)nb;
    for (int k = 0; k < 2; ++k) row[q8t_d(nb, b) + k] = in[k];
    for (int k = 0; k < 16; ++k) {
      row[q8t_qa(nb, b) + k] = in[2 + k];
      row[q8t_qb(nb, b) + k] = in[18 + k];
    }
  }
}

// Q5_K -> Q5_KT: one thread per 16-byte part of the output; 11 parts per superblock in Q5_K's
// order (header, two high-bit halves, eight code runs).
__global__ void repack_q5kt_kernel(int64_t rows, int nsb, const uint8_t* __restrict__ src, uint8_t* __restrict__ dst) {
  const int64_t per_row = 11 * (int64_t)nsb, total = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row;
    const int c = (int)(i % per_row);
    const int t = c / 176, k = c % 176;
    const int m = nsb - 16 * t < 16 ? nsb - 16 * t : 16;
    int from;
    if (k < 3 * m) from = 11 * (k % m) + k / m;  // headers, then the two high-bit halves
    else if (k < 7 * m) from = 11 * ((k - 3 * m) >> 2) + 3 + 2 * ((k - 3 * m) & 3);
    else from = 11 * ((k - 7 * m) >> 2) + 4 + 2 * ((k - 7 * m) & 3);
    const int64_t tile = r * 176 * (int64_t)nsb + 2816 * (int64_t)t;
    *reinterpret_cast<uint4*>(dst + tile + 16 * k) = *reinterpret_cast<const uint4*>(src + tile + 16 * from);
  }
}

hipError_t repack_q5kt_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s) {
  const int64_t total = rows * 11 * (cols >> 8);
  const int64_t nb = (total + 255) / 256;
  const int grid = (int)(nb < 65536 ? nb : 65536);
  hipLaunchKernelGGL(repack_q5kt_kernel, dim3(grid), dim3(256), 0, s, rows, (int)(cols >> 8),
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t repack_q8t_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s) {
  const int64_t total = rows * (cols >> 5);
  const int64_t nb = (total + 255) / 256;
  const int grid = (int)(nb < 65536 ? nb : 65536);
  hipLaunchKernelGGL(repack_q8t_kernel, dim3(grid), dim3(256), 0, s, rows, (int)(cols >> 5),
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t dequant_launch(int fmt, int64_t rows, int64_t cols, const void* blocks, float* w, hipStream_t s) {
  const int64_t total = rows * (cols / 32);
  const int64_t nb = (total + 255) / 256;
  const int grid = (int)(nb < 65536 ? nb : 65536);
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(256), 0, s, fmt, rows, cols,
                     reinterpret_cast<const uint8_t*>(blocks), w);
  return hipGetLastError();
}

// ------------------------------------------------------------ embedding row
__global__ void embed_kernel(int fmt, int64_t n_vocab, int64_t dim, const uint8_t* __restrict__ table,
                             const int32_t* __restrict__ token, float* __restrict__ h,
                             unsigned long long* __restrict__ amax_reset) {
  // row blockIdx.y of a batch of tokens
  const int tok = token[blockIdx.y];
  h += (int64_t)blockIdx.y * dim;
  if (amax_reset && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *amax_reset = 0ull;
  const int be = block_elems(fmt), bb = block_bytes(fmt);
  const int64_t ngroups = dim / 32;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < ngroups; gi += (int64_t)gridDim.x * blockDim.x) {
    float tmp[32];
    if (tok >= 0 && tok < n_vocab) {
      const int64_t c0 = gi * 32;
      dequant_row_group(fmt, table + (int64_t)tok * (dim / be) * bb, dim, c0 / be, (int)((c0 % be) / 32), tmp);
    } else {
      for (int i = 0; i < 32; ++i) tmp[i] = 0.f;
    }
    for (int i = 0; i < 32; ++i) h[gi * 32 + i] = tmp[i];
  }
}

hipError_t embed_launch(int fmt, int64_t n_vocab, int64_t dim, const void* table, const int32_t* token, float* h,
                        unsigned long long* amax_reset, hipStream_t s, int n_tok) {
  const int64_t ng = dim / 32;
  const int grid = (int)((ng + 63) / 64);
  hipLaunchKernelGGL(embed_kernel, dim3(grid, n_tok), dim3(64), 0, s, fmt, n_vocab, dim,
                     reinterpret_cast<const uint8_t*>(table), token, h, amax_reset);
  return hipGetLastError();
}

// ------------------------------------------------------------ RMSNorm
__global__ __launch_bounds__(1024) void rmsnorm_kernel(int64_t n, const float* __restrict__ x,
                                                       const float* __restrict__ g, float eps, float* y) {
  __shared__ float red[16];
  float ss = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) ss += x[i] * x[i];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  const float scale = 1.0f / sqrtf(t / (float)n + eps);
  __syncthreads();
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) y[i] = x[i] * scale * g[i];
}

hipError_t rmsnorm_launch(int64_t n, const float* x, const float* g, float eps, float* y, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(1024), 0, s, n, x, g, eps, y);
  return hipGetLastError();
}

// ------------------------------------------------------------ RoPE
__global__ void rope_kernel(int n_heads, int head_dim, int pos, double theta, float* qk) {
  const int npairs = n_heads * (head_dim / 2);
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < npairs; p += gridDim.x * blockDim.x) {
    const int head = p / (head_dim / 2), i = p % (head_dim / 2);
    const float2 c = rope_cs(theta, pos, i, head_dim);
    const float cs = c.x, sn = c.y;
    float* v = qk + (int64_t)head * head_dim + 2 * i;
    const float x0 = v[0], x1 = v[1];
    v[0] = x0 * cs - x1 * sn;
    v[1] = x0 * sn + x1 * cs;
  }
}

hipError_t rope_launch(int n_heads, int head_dim, int pos, double theta, float* qk, hipStream_t s) {
  const int npairs = n_heads * (head_dim / 2);
  hipLaunchKernelGGL(rope_kernel, dim3((npairs + 255) / 256), dim3(256), 0, s, n_heads, head_dim, pos, theta, qk);
  return hipGetLastError();
}

// ------------------------------------------------------------ SwiGLU
__global__ void swiglu_kernel(int64_t n, const float* gate, const float* up, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float g = gate[i], u = up[i];
    out[i] = g / (1.0f + __expf(-g)) * u;
  }
}

hipError_t swiglu_launch(int64_t n, const float* gate, const float* up, float* out, hipStream_t s) {
  const int64_t nb = (n + 255) / 256;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)(nb < 65536 ? nb : 65536)), dim3(256), 0, s, n, gate, up, out);
  return hipGetLastError();
}

// ------------------------------------------------------------ argmax
__device__ __forceinline__ uint32_t okey(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(1024) void argmax_kernel(int64_t n, const float* __restrict__ v, int32_t* out) {
  __shared__ unsigned long long red[16];
  // row blockIdx.x of a batch of rows of n
  v += (int64_t)blockIdx.x * n;
  out += blockIdx.x;
  unsigned long long best = 0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float x = v[i] != v[i] ? -INFINITY : v[i];
    const unsigned long long key = ((unsigned long long)okey(x) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)i);
    best = key > best ? key : best;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(best, off, 64);
    best = o > best ? o : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long b = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) b = red[i] > b ? red[i] : b;
    *out = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
  }
}

hipError_t argmax_launch(int64_t n, const float* v, int32_t* out, hipStream_t s, int n_rows) {
  hipLaunchKernelGGL(argmax_kernel, dim3(n_rows), dim3(1024), 0, s, n, v, out);
  return hipGetLastError();
}

// The greedy pick of n tokens from their packed (value, index) keys, and the keys' reset
// before a fused LM-head launch folds its maxima into them (a kernel rather than a memset,
// so that callers may capture it in a graph).
__global__ void token_from_key_kernel(const unsigned long long* key, int32_t* token, int n) {
  const int i = (int)threadIdx.x;
  if (i < n) token[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(key[i] & 0xFFFFFFFFull));
}

hipError_t token_from_key_launch(const unsigned long long* key, int32_t* token, hipStream_t s, int n) {
  hipLaunchKernelGGL(token_from_key_kernel, dim3(1), dim3(64), 0, s, key, token, n);
  return hipGetLastError();
}

__global__ void key_reset_kernel(unsigned long long* key, int n) {
  const int i = (int)threadIdx.x;
  if (i < n) key[i] = 0ull;
}

hipError_t key_reset_launch(unsigned long long* key, int n, hipStream_t s) {
  hipLaunchKernelGGL(key_reset_kernel, dim3(1), dim3(64), 0, s, key, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ cosine similarity
// out = sum a b / sqrt(sum a^2 sum b^2), 0 if either vector is zero: the similarity of a
// layer's input and output that cosine-based layer skip ranks layers by (ntransformer
// overview, "Leistung und Caching-Struktur").  One workgroup; the sums in fp64, so the
// result is the exact value to within a few units of fp32 rounding.
__global__ __launch_bounds__(256) void cosine_kernel(int64_t n, const float* __restrict__ a, const float* __restrict__ b,
                                                     float* out) {
  __shared__ double red[3][4];
  double ab = 0.0, aa = 0.0, bb = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    const double x = a[i], y = b[i];
    ab += x * y;
    aa += x * x;
    bb += y * y;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    ab += __shfl_xor(ab, off, 64);
    aa += __shfl_xor(aa, off, 64);
    bb += __shfl_xor(bb, off, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = ab;
    red[1][w] = aa;
    red[2][w] = bb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double s[3];
    for (int k = 0; k < 3; ++k) s[k] = (red[k][0] + red[k][1]) + (red[k][2] + red[k][3]);
    const double den = sqrt(s[1] * s[2]);
    out[0] = den > 0.0 ? (float)(s[0] / den) : 0.f;
  }
}

// ------------------------------------------------------------ read probe
// A plain stream of 16-byte nontemporal loads over a buffer, two in flight per thread, 32
// workgroups of 256 per CU (the fastest of a sweep of 2-32 workgroups per CU, 2-16 loads per
// thread and cached or nontemporal loads: 6.4 TB/s over a 4 GiB buffer, against 5.3-5.8 TB/s
// with cached loads), the data folded into one word per thread that is stored only if it
// equals a value the caller never uses (so the loads cannot be dropped): the achievable HBM
// read rate of the part, next to which the GEMVs' rates can be read.
#ifndef NT_PROBE_WG_PER_CU
#define NT_PROBE_WG_PER_CU 32
#endif
#ifndef NT_PROBE_NT
#define NT_PROBE_NT 1  // nontemporal loads: 6.4 TB/s against 5.75 with cached ones
#endif
#ifndef NT_PROBE_UNROLL
#define NT_PROBE_UNROLL 2
#endif
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n16, uint32_t* sink) {
  constexpr int U = NT_PROBE_UNROLL;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#if NT_PROBE_NT
      v[u] = __builtin_nontemporal_load(p + i + u * stride);
#else
      v[u] = p[i + u * stride];
#endif
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t read_probe_launch(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  int dev = 0, ncu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + 255) / 256;
  const int64_t cap = (int64_t)ncu * NT_PROBE_WG_PER_CU;
  const int grid = (int)(want < cap ? (want > 0 ? want : 1) : cap);
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t cosine_launch(int64_t n, const float* a, const float* b, float* out, hipStream_t s) {
  hipLaunchKernelGGL(cosine_kernel, dim3(1), dim3(256), 0, s, n, a, b, out);
  return hipGetLastError();
}

}  // namespace nt
