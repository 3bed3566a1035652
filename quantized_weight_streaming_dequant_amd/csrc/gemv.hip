// Fused dequantize-and-GEMV over GGML-style block-quantized weights, batch 1, gfx950.
//
// The decode path reads every weight once per token (70B PCIe P2P article,
// blog.hotdry.top, §传统数据路径的性能瓶颈分析), so this kernel is an HBM stream:
//  * each wave owns R consecutive rows (2R for the paired gate/up launch) and walks
//    their blocks left to right; a lane takes one fixed slice of a block per step
//    (a Q8_0/Q4_0 block, a quarter of a Q4_K/Q6_K superblock), loaded with 128-bit
//    global loads at dword-aligned addresses (blocks of 34, 18 and 210 bytes are
//    realigned in registers with v_alignbyte);
//  * codes are unpacked in registers (v_cvt_f32_ubyte* / SDWA sign-extending converts),
//    multiplied with the activation slice held in VGPRs, and scale factors are applied
//    once per 16- or 32-weight group (sum over the group first);
//  * the activation vector (optionally RMS-normalised on the way in) lives in LDS for
//    the whole workgroup, with per-16-column sums for the min/offset terms;
//  * lane partial sums are reduced with cross-lane shuffles;
//  * epilogues fuse the residual add, SwiGLU, RoPE + fp16 KV-cache append, or the
//    greedy argmax, so no extra pass re-reads the output.
// No matrix cores: at batch 1 this is not a dense contraction.
#include "common.h"
#include "gemv.h"

namespace nt {

// ---------------------------------------------------------------- formats

// Q8_0: lane = one 34-byte block (32 weights).  Even and odd blocks are visited in
// separate passes, so every lane of a pass shares the 4-byte phase of its block.
template <int NR>
__device__ __forceinline__ void rows_q8_0(const uint8_t* const (&rowp)[NR], int cols, const float* __restrict__ xl,
                                          const float* __restrict__ xs16, int lane, float (&acc)[NR]) {
  (void)xs16;
  const int nb = cols >> 5;
#pragma unroll 1
  for (int parity = 0; parity < 2; ++parity) {
    const int npar = (nb + 1 - parity) >> 1;
#pragma unroll 1
    for (int s0 = 0; s0 < npar; s0 += 64) {
      const int kk = s0 + lane;
      if (kk >= npar) break;
      const int blk = 2 * kk + parity;
      float x[32];
      const float4* xp = reinterpret_cast<const float4*>(xl + xpad(blk << 5));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = xp[i];
        x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const uint8_t* A = rowp[k] + (size_t)blk * 34;
        const uint32_t phase = (uint32_t)(((uintptr_t)rowp[k] + 2u * parity) & 3u);
        uint32_t q[8];
        uint32_t dbits;
        if (phase == 0) {
          const u32x4 a0 = ld16(A), a1 = ld16(A + 16);
          const uint32_t t = ld2(A + 32);
          dbits = a0.x;
          q[0] = __builtin_amdgcn_alignbyte(a0.y, a0.x, 2);
          q[1] = __builtin_amdgcn_alignbyte(a0.z, a0.y, 2);
          q[2] = __builtin_amdgcn_alignbyte(a0.w, a0.z, 2);
          q[3] = __builtin_amdgcn_alignbyte(a1.x, a0.w, 2);
          q[4] = __builtin_amdgcn_alignbyte(a1.y, a1.x, 2);
          q[5] = __builtin_amdgcn_alignbyte(a1.z, a1.y, 2);
          q[6] = __builtin_amdgcn_alignbyte(a1.w, a1.z, 2);
          q[7] = __builtin_amdgcn_alignbyte(t, a1.w, 2);
        } else {
          const uint32_t e = ld4(A - 2);
          const u32x4 a0 = ld16(A + 2), a1 = ld16(A + 18);
          dbits = e >> 16;
          q[0] = a0.x; q[1] = a0.y; q[2] = a0.z; q[3] = a0.w;
          q[4] = a1.x; q[5] = a1.y; q[6] = a1.z; q[7] = a1.w;
        }
        float s0a = 0.f, s1a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          s0a += sb0(q[i]) * x[4 * i] + sb1(q[i]) * x[4 * i + 1] + sb2(q[i]) * x[4 * i + 2] + sb3(q[i]) * x[4 * i + 3];
          s1a += sb0(q[i + 1]) * x[4 * i + 4] + sb1(q[i + 1]) * x[4 * i + 5] + sb2(q[i + 1]) * x[4 * i + 6] +
                 sb3(q[i + 1]) * x[4 * i + 7];
        }
        acc[k] += h2f(dbits) * (s0a + s1a);
      }
    }
  }
}

// Q4_0: lane = one 18-byte block; w = d (n - 8) = d n - 8 d, so the block sum is
// d (sum n x - 8 sum x) with sum x over the block's 32 columns taken from LDS.
template <int NR>
__device__ __forceinline__ void rows_q4_0(const uint8_t* const (&rowp)[NR], int cols, const float* __restrict__ xl,
                                          const float* __restrict__ xs16, int lane, float (&acc)[NR]) {
  const int nb = cols >> 5;
#pragma unroll 1
  for (int parity = 0; parity < 2; ++parity) {
    const int npar = (nb + 1 - parity) >> 1;
#pragma unroll 1
    for (int s0 = 0; s0 < npar; s0 += 64) {
      const int kk = s0 + lane;
      if (kk >= npar) break;
      const int blk = 2 * kk + parity;
      float x[32];
      const float4* xp = reinterpret_cast<const float4*>(xl + xpad(blk << 5));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 v = xp[i];
        x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
      }
      const float xsum = xs16[2 * blk] + xs16[2 * blk + 1];
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const uint8_t* A = rowp[k] + (size_t)blk * 18;
        const uint32_t phase = (uint32_t)(((uintptr_t)rowp[k] + 2u * parity) & 3u);
        uint32_t q[4];
        uint32_t dbits;
        if (phase == 0) {
          const u32x4 a0 = ld16(A);
          const uint32_t t = ld2(A + 16);
          dbits = a0.x;
          q[0] = __builtin_amdgcn_alignbyte(a0.y, a0.x, 2);
          q[1] = __builtin_amdgcn_alignbyte(a0.z, a0.y, 2);
          q[2] = __builtin_amdgcn_alignbyte(a0.w, a0.z, 2);
          q[3] = __builtin_amdgcn_alignbyte(t, a0.w, 2);
        } else {
          const uint32_t e = ld4(A - 2);
          const u32x4 a0 = ld16(A + 2);
          dbits = e >> 16;
          q[0] = a0.x; q[1] = a0.y; q[2] = a0.z; q[3] = a0.w;
        }
        float slo = 0.f, shi = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = opaque(q[i] & 0x0F0F0F0Fu);
          const uint32_t hi = opaque((q[i] >> 4) & 0x0F0F0F0Fu);
          slo += ub0(lo) * x[4 * i] + ub1(lo) * x[4 * i + 1] + ub2(lo) * x[4 * i + 2] + ub3(lo) * x[4 * i + 3];
          shi += ub0(hi) * x[16 + 4 * i] + ub1(hi) * x[17 + 4 * i] + ub2(hi) * x[18 + 4 * i] + ub3(hi) * x[19 + 4 * i];
        }
        acc[k] += h2f(dbits) * ((slo + shi) - 8.f * xsum);
      }
    }
  }
}

// Q4_K: lane = quarter g of a 144-byte superblock: the 32 bytes of nibbles at 16 + 32 g,
// whose low nibbles are sub-block 2g and high nibbles sub-block 2g+1 (64 weights).
// w = d sc q - dmin m: per sub-block  d sc (sum q x) - dmin m (sum x).
template <int NR>
__device__ __forceinline__ void rows_q4_k(const uint8_t* const (&rowp)[NR], int cols, const float* __restrict__ xl,
                                          const float* __restrict__ xs16, int lane, float (&acc)[NR]) {
  const int nsb = cols >> 8;
  const int g = lane & 3;
  const bool upper = g >= 2;            // sub-blocks 4..7 keep their scale bits split
  const uint32_t bsh = (uint32_t)(g & 1) * 16u;
#pragma unroll 1
  for (int s0 = 0; s0 < nsb; s0 += 16) {
    const int sb = s0 + (lane >> 2);
    if (sb >= nsb) break;
    const int c0 = (sb << 8) + (g << 6);
    float x[64];
    const float4* xp = reinterpret_cast<const float4*>(xl + xpad(c0));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 v = xp[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
    const float xa = xs16[(c0 >> 4)] + xs16[(c0 >> 4) + 1];
    const float xb = xs16[(c0 >> 4) + 2] + xs16[(c0 >> 4) + 3];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint8_t* p = rowp[k] + (size_t)sb * 144;
      const u32x4 hd = ld16(p);
      const u32x4 qa = ld16(p + 16 + 32 * g);
      const u32x4 qb = ld16(p + 32 + 32 * g);
      const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
      float slo0 = 0.f, slo1 = 0.f, shi0 = 0.f, shi1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t lo0 = opaque(q[i] & 0x0F0F0F0Fu), hi0 = opaque((q[i] >> 4) & 0x0F0F0F0Fu);
        const uint32_t lo1 = opaque(q[i + 1] & 0x0F0F0F0Fu), hi1 = opaque((q[i + 1] >> 4) & 0x0F0F0F0Fu);
        slo0 += ub0(lo0) * x[4 * i] + ub1(lo0) * x[4 * i + 1] + ub2(lo0) * x[4 * i + 2] + ub3(lo0) * x[4 * i + 3];
        slo1 += ub0(lo1) * x[4 * i + 4] + ub1(lo1) * x[4 * i + 5] + ub2(lo1) * x[4 * i + 6] + ub3(lo1) * x[4 * i + 7];
        shi0 += ub0(hi0) * x[32 + 4 * i] + ub1(hi0) * x[33 + 4 * i] + ub2(hi0) * x[34 + 4 * i] + ub3(hi0) * x[35 + 4 * i];
        shi1 += ub0(hi1) * x[36 + 4 * i] + ub1(hi1) * x[37 + 4 * i] + ub2(hi1) * x[38 + 4 * i] + ub3(hi1) * x[39 + 4 * i];
      }
      // 6-bit scale/min of sub-blocks 2g and 2g+1: bytes 2(g&1) and 2(g&1)+1 of the
      // three scale words (bytes 4..7, 8..11, 12..15 of the block).
      const uint32_t Y = hd.y >> bsh, Z = hd.z >> bsh, W = hd.w >> bsh;
      const uint32_t sca = upper ? ((W & 15u) | ((Y >> 2) & 48u)) : (Y & 63u);
      const uint32_t scb = upper ? (((W >> 8) & 15u) | ((Y >> 10) & 48u)) : ((Y >> 8) & 63u);
      const uint32_t ma = upper ? (((W >> 4) & 15u) | ((Z >> 2) & 48u)) : (Z & 63u);
      const uint32_t mb = upper ? (((W >> 12) & 15u) | ((Z >> 10) & 48u)) : ((Z >> 8) & 63u);
      const float d = h2f(hd.x), dmin = h2f(hd.x >> 16);
      acc[k] += d * ((float)sca * (slo0 + slo1) + (float)scb * (shi0 + shi1)) - dmin * ((float)ma * xa + (float)mb * xb);
    }
  }
}

// Q6_K: lane = quarter (h, half) of a 210-byte superblock: weights 128h + 32t + 16half + [0,16)
// for t = 0..3 (64 weights).  Their low nibbles sit in 16-byte runs of the low-nibble
// array (t even: low nibbles, t odd: next run; t >= 2: high nibbles), their two high bits
// in one 16-byte run of the high-bit array, their scales in bytes 2t + half of an 8-byte
// group.  w = d s (q - 32): per 16-weight group  d s (sum q x - 32 sum x).
// Even and odd superblocks are visited in separate passes (210 = 2 mod 4).
__device__ __forceinline__ uint32_t q6_codes(uint32_t lw, uint32_t hw, int t) {
  const uint32_t lo = (t < 2) ? (lw & 0x0F0F0F0Fu) : ((lw >> 4) & 0x0F0F0F0Fu);
  uint32_t hb;
  if (t == 0) hb = (hw << 4) & 0x30303030u;
  else if (t == 1) hb = (hw << 2) & 0x30303030u;
  else if (t == 2) hb = hw & 0x30303030u;
  else hb = (hw >> 2) & 0x30303030u;
  return opaque(lo | hb);
}

template <int NR>
__device__ __forceinline__ void rows_q6_k(const uint8_t* const (&rowp)[NR], int cols, const float* __restrict__ xl,
                                          const float* __restrict__ xs16, int lane, float (&acc)[NR]) {
  const int nsb = cols >> 8;
  const int quarter = lane & 3, h = quarter >> 1, half = quarter & 1;
  const int offL0 = 64 * h + 16 * half, offL1 = offL0 + 32, offH = 128 + 32 * h + 16 * half, offS = 192 + 8 * h;
#pragma unroll 1
  for (int parity = 0; parity < 2; ++parity) {
    const int npar = (nsb + 1 - parity) >> 1;
#pragma unroll 1
    for (int s0 = 0; s0 < npar; s0 += 16) {
      const int kk = s0 + (lane >> 2);
      if (kk >= npar) break;
      const int sb = 2 * kk + parity;
      const int cb = (sb << 8) + 128 * h + 16 * half;
      float x[64];
      float xsum[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float4* xp = reinterpret_cast<const float4*>(xl + xpad(cb + 32 * t));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = xp[i];
          x[16 * t + 4 * i] = v.x; x[16 * t + 4 * i + 1] = v.y; x[16 * t + 4 * i + 2] = v.z; x[16 * t + 4 * i + 3] = v.w;
        }
        xsum[t] = xs16[(cb + 32 * t) >> 4];
      }
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const uint8_t* A = rowp[k] + (size_t)sb * 210;
        const uint32_t phase = (uint32_t)(((uintptr_t)rowp[k] + 2u * parity) & 3u);
        u32x4 L0, L1, H;
        u32x2 S;
        if (phase == 0) {
          L0 = ld16(A + offL0); L1 = ld16(A + offL1); H = ld16(A + offH); S = ld8(A + offS);
        } else {
          L0 = ld16_off2(A + offL0); L1 = ld16_off2(A + offL1); H = ld16_off2(A + offH); S = ld8_off2(A + offS);
        }
        const float d = h2f(ld2(A + 208));
        const uint32_t Lw0[4] = {L0.x, L0.y, L0.z, L0.w};
        const uint32_t Lw1[4] = {L1.x, L1.y, L1.z, L1.w};
        const uint32_t Hw[4] = {H.x, H.y, H.z, H.w};
        float tot = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float s = 0.f, s2 = 0.f;
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const uint32_t c0 = q6_codes((t & 1) ? Lw1[i] : Lw0[i], Hw[i], t);
            const uint32_t c1 = q6_codes((t & 1) ? Lw1[i + 1] : Lw0[i + 1], Hw[i + 1], t);
            s += ub0(c0) * x[16 * t + 4 * i] + ub1(c0) * x[16 * t + 4 * i + 1] + ub2(c0) * x[16 * t + 4 * i + 2] +
                 ub3(c0) * x[16 * t + 4 * i + 3];
            s2 += ub0(c1) * x[16 * t + 4 * i + 4] + ub1(c1) * x[16 * t + 4 * i + 5] + ub2(c1) * x[16 * t + 4 * i + 6] +
                  ub3(c1) * x[16 * t + 4 * i + 7];
          }
          // sub-scale of this 16-weight group: byte 2t + half of the 8 scale bytes
          const uint32_t sw = (t < 2) ? S.x : S.y;
          const float sc = (float)(int8_t)((sw >> (8 * (2 * (t & 1) + half))) & 0xFFu);
          tot += sc * ((s + s2) - 32.f * xsum[t]);
        }
        acc[k] += d * tot;
      }
    }
  }
}

// ---------------------------------------------------------------- kernel

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Stage x (optionally RMS-normalised) into LDS and the sums of every 16 columns.
__device__ __forceinline__ void stage_x(const GemvArgs& a, float* xl, float* xs16, float* red) {
  const int cols = a.cols;
  float scale = 1.f;
  if (a.gain) {
    float ss = 0.f;
    for (int c = threadIdx.x * 4; c < cols; c += blockDim.x * 4) {
      const float4 v = *reinterpret_cast<const float4*>(a.x + c);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = block_sum(ss, red);
    scale = 1.0f / sqrtf(ss / (float)cols + a.eps);
  }
  for (int gi = threadIdx.x; gi < (cols >> 4); gi += blockDim.x) {
    const float4* src = reinterpret_cast<const float4*>(a.x + gi * 16);
    float4 v[4] = {src[0], src[1], src[2], src[3]};
    if (a.gain) {
      const float4* gp = reinterpret_cast<const float4*>(a.gain + gi * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 gg = gp[i];
        v[i].x = v[i].x * scale * gg.x; v[i].y = v[i].y * scale * gg.y;
        v[i].z = v[i].z * scale * gg.z; v[i].w = v[i].w * scale * gg.w;
      }
    }
    float4* dst = reinterpret_cast<float4*>(xl + xpad(gi * 16));
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dst[i] = v[i];
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    xs16[gi] = s;
  }
  __syncthreads();
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Map an fp32 value to a uint32 whose unsigned order is the float order.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int FMTMASK, int R, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(const GemvArgs a) {
  extern __shared__ float4 smem4[];
  float* xl = reinterpret_cast<float*>(smem4);
  float* xs16 = xl + xpad_len(a.cols);
  float* red = xs16 + (a.cols >> 4);
  stage_x(a, xl, xs16, red);

  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int tile = blockIdx.x;
  int s = 0;
  if (a.nseg > 1 && tile >= a.seg[1].tile0) s = 1;
  if (a.nseg > 2 && tile >= a.seg[2].tile0) s = 2;
  const GemvSeg sg = a.seg[s];
  const int row0 = (tile - sg.tile0) * (NW * R) + wave * R;
  if (row0 >= sg.rows) return;  // no barrier follows

  const uint8_t* rowp[NR];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int r = min(row0 + k, sg.rows - 1);  // past-the-end rows re-read the last row; results dropped
    rowp[k] = sg.w + (size_t)r * sg.row_bytes;
    if constexpr (EPI == EPI_SWIGLU) rowp[R + k] = a.seg[1].w + (size_t)r * sg.row_bytes;
  }
  float acc[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) acc[k] = 0.f;

  switch (sg.fmt) {
    case FMT_Q8_0:
      if constexpr ((FMTMASK >> FMT_Q8_0) & 1) rows_q8_0<NR>(rowp, a.cols, xl, xs16, lane, acc);
      break;
    case FMT_Q4_0:
      if constexpr ((FMTMASK >> FMT_Q4_0) & 1) rows_q4_0<NR>(rowp, a.cols, xl, xs16, lane, acc);
      break;
    case FMT_Q4_K:
      if constexpr ((FMTMASK >> FMT_Q4_K) & 1) rows_q4_k<NR>(rowp, a.cols, xl, xs16, lane, acc);
      break;
    default:
      if constexpr ((FMTMASK >> FMT_Q6_K) & 1) rows_q6_k<NR>(rowp, a.cols, xl, xs16, lane, acc);
      break;
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) acc[k] = wave_sum(acc[k]);

  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS) {
    if (lane < R && row0 + lane < sg.rows) {
      float v = acc[0];
#pragma unroll
      for (int k = 1; k < R; ++k) v = (lane == k) ? acc[k] : v;
      a.y[row0 + lane] = v;
    }
    if constexpr (EPI == EPI_LOGITS) {
      if (lane == 0) {
        unsigned long long best = 0;
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const int r = row0 + k;
          if (r < sg.rows) {
            const float v = acc[k] != acc[k] ? -INFINITY : acc[k];  // NaN never wins
            const unsigned long long key =
                ((unsigned long long)order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)r);
            best = key > best ? key : best;
          }
        }
        atomicMax(a.amax, best);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    if (lane < R && row0 + lane < sg.rows) {
      float v = acc[0];
#pragma unroll
      for (int k = 1; k < R; ++k) v = (lane == k) ? acc[k] : v;
      const int r = row0 + lane;
      const float o = a.resid[r] + v;
      a.y[r] = o;
      if (a.y2) a.y2[r] = o;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (lane < R && row0 + lane < sg.rows) {
      float g = acc[0], u = acc[R];
#pragma unroll
      for (int k = 1; k < R; ++k) {
        g = (lane == k) ? acc[k] : g;
        u = (lane == k) ? acc[R + k] : u;
      }
      a.y[row0 + lane] = silu_mul(g, u);
    }
  } else if constexpr (EPI == EPI_QKV) {
    // rows come in RoPE pairs (2i, 2i+1) inside one head of 128; R is even
    constexpr int HD = 128;
    const int npair = R / 2;
    if (lane < npair) {
      float y0 = acc[0], y1 = acc[1];
#pragma unroll
      for (int p = 1; p < R / 2; ++p) {
        y0 = (lane == p) ? acc[2 * p] : y0;
        y1 = (lane == p) ? acc[2 * p + 1] : y1;
      }
      const int r = row0 + 2 * lane;
      if (r < sg.rows) {
        const int head = r / HD, dd = r % HD;
        if (s < 2) {
          const int i = dd >> 1;
          // angle pos * theta^(-2i/HD) formed and reduced to [-pi, pi] in fp64
          const double f = pow(a.rope_theta, -2.0 * (double)i / (double)HD);
          double ang = (double)a.pos * f;
          ang -= 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
          float sn, cs;
          sincosf((float)ang, &sn, &cs);
          const float r0 = y0 * cs - y1 * sn;
          const float r1 = y0 * sn + y1 * cs;
          if (s == 0) {
            a.q_out[r] = r0;
            a.q_out[r + 1] = r1;
          } else {
            uint16_t* kp = a.k_cache + ((size_t)head * a.max_ctx + a.pos) * HD + dd;
            kp[0] = f2h_rne(r0);
            kp[1] = f2h_rne(r1);
          }
        } else {
          uint16_t* vp = a.v_cache + ((size_t)head * a.max_ctx + a.pos) * HD + dd;
          vp[0] = f2h_rne(y0);
          vp[1] = f2h_rne(y1);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

GemvPlan gemv_plan(int epi, int cols) {
  GemvPlan p;
  // the paired gate/up launch already carries two rows per wave slot
  p.rows_per_wave = (epi == EPI_SWIGLU) ? 1 : 2;
  p.waves = 8;
  p.lds_bytes = sizeof(float) * (size_t)(xpad_len(cols) + (cols >> 4) + 16);
  return p;
}

int gemv_tiles(const GemvPlan& p, int rows) {
  const int per = p.rows_per_wave * p.waves;
  return (rows + per - 1) / per;
}

template <int FMTMASK, int NW, int EPI>
static hipError_t launch_one(const GemvPlan& plan, int n_tiles, const GemvArgs& a, hipStream_t s) {
  constexpr int R = (EPI == EPI_SWIGLU) ? 1 : 2;
  auto kern = gemv_kernel<FMTMASK, R, NW, EPI>;
  static bool attr_set = false;  // benign race: idempotent attribute
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(n_tiles), dim3(NW * 64), plan.lds_bytes, s, a);
  return hipGetLastError();
}

template <int FMTMASK, int EPI>
static hipError_t launch_nw(const GemvPlan& plan, int n_tiles, const GemvArgs& a, hipStream_t s) {
  if (plan.waves != 8) return hipErrorInvalidConfiguration;
  return launch_one<FMTMASK, 8, EPI>(plan, n_tiles, a, s);
}

template <int EPI>
static hipError_t launch_mask(int fmt_mask, const GemvPlan& plan, int n_tiles, const GemvArgs& a, hipStream_t s) {
  switch (fmt_mask) {
    case 1 << FMT_Q8_0: return launch_nw<1 << FMT_Q8_0, EPI>(plan, n_tiles, a, s);
    case 1 << FMT_Q4_0: return launch_nw<1 << FMT_Q4_0, EPI>(plan, n_tiles, a, s);
    case 1 << FMT_Q4_K: return launch_nw<1 << FMT_Q4_K, EPI>(plan, n_tiles, a, s);
    case 1 << FMT_Q6_K: return launch_nw<1 << FMT_Q6_K, EPI>(plan, n_tiles, a, s);
    case (1 << FMT_Q4_K) | (1 << FMT_Q6_K): return launch_nw<(1 << FMT_Q4_K) | (1 << FMT_Q6_K), EPI>(plan, n_tiles, a, s);
    default: return launch_nw<15, EPI>(plan, n_tiles, a, s);
  }
}

hipError_t gemv_launch(int fmt_mask, int epi, const GemvPlan& plan, int n_tiles, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_mask<EPI_STORE>(fmt_mask, plan, n_tiles, a, s);
    case EPI_RESID: return launch_mask<EPI_RESID>(fmt_mask, plan, n_tiles, a, s);
    case EPI_SWIGLU: return launch_mask<EPI_SWIGLU>(fmt_mask, plan, n_tiles, a, s);
    case EPI_QKV: return launch_mask<EPI_QKV>(fmt_mask, plan, n_tiles, a, s);
    default: return launch_mask<EPI_LOGITS>(fmt_mask, plan, n_tiles, a, s);
  }
}

}  // namespace nt
