// Fused dequantize-and-GEMV over GGML-style block-quantized weights, batch 1, gfx950.
//
// The decode path reads every weight once per token (70B PCIe P2P article,
// blog.hotdry.top, §传统数据路径的性能瓶颈分析), so this kernel is an HBM stream with a
// tight ALU budget (about 2.8 VALU lane-operations per 4.5-bit weight at 8 TB/s):
//  * persistent workgroups, as many as stay resident: each stages the activation vector
//    x (optionally RMS-normalised on the way in) into LDS once, with per-16-column sums;
//  * the work is groups of R consecutive rows (2R rows for the paired gate/up launch)
//    dealt round-robin to every wave of the launch, so waves finish together; a wave
//    walks its rows' blocks in steps, a lane taking one fixed slice of a block per step
//    (a Q8_0/Q4_0 block, a quarter of a Q4_K/Q6_K superblock) with dword-aligned 128-bit
//    loads, and the loads of the next step are in flight while the current one computes;
//  * blocks of 34, 18 and 210 bytes sit at 2-byte phases: the step order visits even and
//    odd blocks separately so that the phase is uniform per row and step, and a scalar
//    branch realigns with v_alignbyte;
//  * 4- and 6-bit codes become exact fp16 values 1024 + q (or 1024 + 16q) by OR-ing the
//    exponent bits in, and v_fma_mix_f32 multiplies them with the fp32 activation in one
//    instruction; the 1024 offsets come back out through the per-16-column sums of x;
//  * scale factors are applied once per 16 or 32 weights, lane sums are reduced with
//    cross-lane shuffles, and epilogues fuse the residual add, SwiGLU, RoPE + fp16 KV
//    append, or the greedy argmax.
// No matrix cores: at batch 1 this is not a dense contraction.
#include "common.h"
#include "gemv.h"

namespace nt {

// ------------------------------------------------------------------ helpers

constexpr uint32_t F16_1024 = 0x64006400u;  // two fp16 1024.0: OR a small integer into the mantissa

__device__ __forceinline__ float lo_h(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v & 0xFFFFu))); }
__device__ __forceinline__ float hi_h(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v >> 16))); }

// Launch-geometry and load-policy defaults (overridable at build time).
#ifndef NT_GEMV_WG_PER_CU_MAX
#define NT_GEMV_WG_PER_CU_MAX 0  // 0: as many workgroups per CU as stay resident
#endif
#ifndef NT_GEMV_NONTEMPORAL
#define NT_GEMV_NONTEMPORAL 0
#endif

// Weight loads.  Nontemporal loads were measured slower on every GEMV shape here (by
// 10-30%), so plain cached loads are the default.
#if NT_GEMV_NONTEMPORAL
__device__ __forceinline__ u32x4 wld16(const uint8_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
__device__ __forceinline__ uint32_t wld4(const uint8_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }
__device__ __forceinline__ uint32_t wld2(const uint8_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)); }
#else
__device__ __forceinline__ u32x4 wld16(const uint8_t* p) { return ld16(p); }
__device__ __forceinline__ uint32_t wld4(const uint8_t* p) { return ld4(p); }
__device__ __forceinline__ uint32_t wld2(const uint8_t* p) { return ld2(p); }
#endif

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// (a & b) | c, written so that it becomes one v_and_or_b32.  VOP3 encodings take no
// literal constants and at most one scalar operand on this target, so with two constant
// masks the compiler would split it into an AND and an OR; callers pass masks that were
// first moved into VGPRs with vreg().
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) { return (a & b) | c; }
__device__ __forceinline__ uint32_t vreg(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Nibble-to-fp16 masks: low nibbles of bytes 0 and 2, high nibbles of bytes 0 and 2.
constexpr uint32_t NIB_LO = 0x000F000Fu, NIB_HI = 0x00F000F0u;
// v_perm_b32 selectors: result bytes {src1.b0, src0.b1, src1.b2, src0.b3} (resp. b1, b3 of
// src1); selector values 0-3 pick src1 bytes, 4-7 src0 bytes
constexpr uint32_t PERM_B02 = 0x07020500u, PERM_B13 = 0x07030501u;

// ------------------------------------------------------------------ formats
//
// Each format provides:
//   Raw                          registers of one row's slice for one step
//   steps(cols)                  steps per row
//   load(rowp, cols, step, lane) issue the global loads of one row's slice
//   fma(raw[NR], ..., acc[NR])   consume them: acc[k] += this step's part of row k

// Q8_0: lane = one 34-byte block; steps visit the even blocks, then the odd ones.
struct Q8_0F {
  struct Raw {
    uint32_t w[9];
    uint32_t ph;
  };
  static __device__ __forceinline__ int steps(int cols) {
    const int nb = cols >> 5;
    return ((nb + 1) / 2 + 63) / 64 + (nb / 2 + 63) / 64;
  }
  static __device__ __forceinline__ int block_of(int cols, int step, int lane, bool& ok) {
    const int nb = cols >> 5;
    const int se = ((nb + 1) / 2 + 63) / 64;
    const int parity = step >= se ? 1 : 0;
    const int k = (step - parity * se) * 64 + lane;
    const int blk = 2 * k + parity;
    ok = blk < nb;
    return blk;
  }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    bool ok;
    const int blk = block_of(cols, step, lane, ok);
    Raw r;
    const uint8_t* A = rowp + (size_t)(ok ? blk : (blk & 1)) * 34;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));  // the same for every lane of the step
    if (r.ph == 0) {
      const u32x4 a = wld16(A), b = wld16(A + 16);
      r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
      r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
      r.w[8] = wld2(A + 32);
    } else {
      r.w[0] = wld4(A - 2);
      const u32x4 a = wld16(A + 2), b = wld16(A + 18);
      r.w[1] = a.x; r.w[2] = a.y; r.w[3] = a.z; r.w[4] = a.w;
      r.w[5] = b.x; r.w[6] = b.y; r.w[7] = b.z; r.w[8] = b.w;
    }
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane,
                                             const float* __restrict__ xl, const float* __restrict__ xs16,
                                             float (&acc)[NR]) {
    (void)xs16;
    bool ok;
    const int blk = block_of(cols, step, lane, ok);
    if (!ok) return;
    const float4* xp = reinterpret_cast<const float4*>(xl + xpad(blk << 5));
    float s[NR];
    uint32_t q[NR][8];
    float d[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      s[k] = 0.f;
      if (raw[k].ph == 0) {
        d[k] = h2f(raw[k].w[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = __builtin_amdgcn_alignbyte(raw[k].w[i + 1], raw[k].w[i], 2);
      } else {
        d[k] = h2f(raw[k].w[0] >> 16);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = raw[k].w[i + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 xv = xp[i];
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        s[k] += sb0(q[k][i]) * xv.x;
        s[k] += sb1(q[k][i]) * xv.y;
        s[k] += sb2(q[k][i]) * xv.z;
        s[k] += sb3(q[k][i]) * xv.w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] += d[k] * s[k];
  }
};

// Q4_0: lane = one 18-byte block; weights 0..15 are the low nibbles, 16..31 the high ones.
struct Q4_0F {
  struct Raw {
    uint32_t w[5];
    uint32_t ph;
  };
  static __device__ __forceinline__ int steps(int cols) { return Q8_0F::steps(cols); }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    bool ok;
    const int blk = Q8_0F::block_of(cols, step, lane, ok);
    Raw r;
    const uint8_t* A = rowp + (size_t)(ok ? blk : (blk & 1)) * 18;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));
    if (r.ph == 0) {
      const u32x4 a = wld16(A);
      r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
      r.w[4] = wld2(A + 16);
    } else {
      r.w[0] = wld4(A - 2);
      const u32x4 a = wld16(A + 2);
      r.w[1] = a.x; r.w[2] = a.y; r.w[3] = a.z; r.w[4] = a.w;
    }
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane,
                                             const float* __restrict__ xl, const float* __restrict__ xs16,
                                             float (&acc)[NR]) {
    bool ok;
    const int blk = Q8_0F::block_of(cols, step, lane, ok);
    if (!ok) return;
    const float4* xp = reinterpret_cast<const float4*>(xl + xpad(blk << 5));
    const float xlo = xs16[2 * blk], xhi = xs16[2 * blk + 1];
    float slo[NR], shi[NR], d[NR];
    uint32_t q[NR][4];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      slo[k] = shi[k] = 0.f;
      if (raw[k].ph == 0) {
        d[k] = h2f(raw[k].w[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[k][i] = __builtin_amdgcn_alignbyte(raw[k].w[i + 1], raw[k].w[i], 2);
      } else {
        d[k] = h2f(raw[k].w[0] >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[k][i] = raw[k].w[i + 1];
      }
    }
    const uint32_t mlo = vreg(NIB_LO), mhi = vreg(NIB_HI), m1024 = vreg(F16_1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xa = xp[i], xb = xp[4 + i];  // columns 4i.. (low nibbles), 16+4i.. (high nibbles)
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const uint32_t v = q[k][i], u = v >> 8;
        const uint32_t p0 = and_or(v, mlo, m1024), p1 = and_or(v, mhi, m1024);
        const uint32_t p2 = and_or(u, mlo, m1024), p3 = and_or(u, mhi, m1024);
        slo[k] += lo_h(p0) * xa.x;
        slo[k] += lo_h(p2) * xa.y;
        slo[k] += hi_h(p0) * xa.z;
        slo[k] += hi_h(p2) * xa.w;
        shi[k] += lo_h(p1) * xb.x;
        shi[k] += lo_h(p3) * xb.y;
        shi[k] += hi_h(p1) * xb.z;
        shi[k] += hi_h(p3) * xb.w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // slo = sum (1024 + n) x, shi = sum (1024 + 16 n) x;  w = d (n - 8)
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const float sn = (slo[k] - 1024.f * xlo) + 0.0625f * (shi[k] - 1024.f * xhi);
      acc[k] += d[k] * (sn - 8.f * (xlo + xhi));
    }
  }
};

// Q4_K: lane = quarter g of a 144-byte superblock: the 32 nibble bytes at 16 + 32 g, whose
// low nibbles are sub-block 2g and high nibbles sub-block 2g+1 (64 weights); 16 superblocks
// per step.  w = d sc q - dmin m, summed per sub-block as d sc (sum q x) - dmin m (sum x).
struct Q4_KF {
  struct Raw {
    u32x4 hd, qa, qb;
  };
  static __device__ __forceinline__ int steps(int cols) { return ((cols >> 8) + 15) / 16; }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    const int nsb = cols >> 8;
    int sb = step * 16 + (lane >> 2);
    sb = sb < nsb ? sb : 0;
    const int g = lane & 3;
    const uint8_t* p = rowp + (size_t)sb * 144;
    Raw r;
    r.hd = wld16(p);
    r.qa = wld16(p + 16 + 32 * g);
    r.qb = wld16(p + 32 + 32 * g);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane,
                                             const float* __restrict__ xl, const float* __restrict__ xs16,
                                             float (&acc)[NR]) {
    const int nsb = cols >> 8;
    const int sb = step * 16 + (lane >> 2);
    if (sb >= nsb) return;
    const int g = lane & 3;
    const int c0 = (sb << 8) + (g << 6);
    const float4* xp = reinterpret_cast<const float4*>(xl + xpad(c0));
    const float xa = xs16[c0 >> 4] + xs16[(c0 >> 4) + 1];
    const float xb = xs16[(c0 >> 4) + 2] + xs16[(c0 >> 4) + 3];
    float slo[NR], shi[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) slo[k] = shi[k] = 0.f;
    const uint32_t mlo = vreg(NIB_LO), mhi = vreg(NIB_HI), m1024 = vreg(F16_1024);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // nibble bytes 4i..4i+3: low nibbles -> columns c0+4i.., high nibbles -> c0+32+4i..
      const float4 xv = xp[i], xw = xp[8 + i];
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        const uint32_t v = (i < 4) ? raw[k].qa[i & 3] : raw[k].qb[i & 3];
        const uint32_t u = v >> 8;
        const uint32_t p0 = and_or(v, mlo, m1024), p1 = and_or(v, mhi, m1024);
        const uint32_t p2 = and_or(u, mlo, m1024), p3 = and_or(u, mhi, m1024);
        slo[k] += lo_h(p0) * xv.x;
        slo[k] += lo_h(p2) * xv.y;
        slo[k] += hi_h(p0) * xv.z;
        slo[k] += hi_h(p2) * xv.w;
        shi[k] += lo_h(p1) * xw.x;
        shi[k] += lo_h(p3) * xw.y;
        shi[k] += hi_h(p1) * xw.z;
        shi[k] += hi_h(p3) * xw.w;
      }
      // keep each chunk's LDS reads next to their use: hoisting all of them costs 64 VGPRs
      __builtin_amdgcn_sched_barrier(0);
    }
    // 6-bit scale/min of sub-blocks 2g and 2g+1 from the scale words Y (bytes 4..7), Z (8..11),
    // W (12..15).  Sub-blocks 0..3: scale = bits of Y, min = bits of Z, at byte 2(g&1) (and +1).
    // Sub-blocks 4..7: low four bits in W (scale: low nibble, min: high nibble), top two bits
    // in bits 6..7 of the same bytes of Y (scale) and Z (min).  All lane-constant field
    // positions, so each field is one or two bit-field extracts (width 0 extracts 0).
    const bool upper = g >= 2;
    const uint32_t o = 16u * (uint32_t)(g & 1);
    const uint32_t wl = upper ? 4u : 6u, wh = upper ? 2u : 0u, om = upper ? o + 4u : o;
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint32_t Y = raw[k].hd.y, Z = raw[k].hd.z, W = raw[k].hd.w;
      const uint32_t srcS = upper ? W : Y, srcM = upper ? W : Z;
      const uint32_t sca = __builtin_amdgcn_ubfe(srcS, o, wl) | (__builtin_amdgcn_ubfe(Y, o + 6u, wh) << 4);
      const uint32_t scb = __builtin_amdgcn_ubfe(srcS, o + 8u, wl) | (__builtin_amdgcn_ubfe(Y, o + 14u, wh) << 4);
      const uint32_t ma = __builtin_amdgcn_ubfe(srcM, om, wl) | (__builtin_amdgcn_ubfe(Z, o + 6u, wh) << 4);
      const uint32_t mb = __builtin_amdgcn_ubfe(srcM, om + 8u, wl) | (__builtin_amdgcn_ubfe(Z, o + 14u, wh) << 4);
      const float d = h2f(raw[k].hd.x), dmin = h2f(raw[k].hd.x >> 16);
      // slo = sum (1024 + q) x over sub-block 2g, shi = sum (1024 + 16 q) x over 2g+1
      const float A = slo[k] - 1024.f * xa;
      const float B = shi[k] - 1024.f * xb;
      acc[k] += (d * (float)sca) * A;
      acc[k] += (d * 0.0625f * (float)scb) * B;
      acc[k] -= dmin * ((float)ma * xa + (float)mb * xb);
    }
  }
};

// Q6_K: lane = one eighth of a 210-byte superblock, (h, tp, half) with h, tp, half in {0,1}:
// the 16 low-nibble bytes at 64h + 32tp + 16half (the next eight lanes read the next 128
// bytes), the 16 high-bit bytes at 128 + 32h + 16half, and the scale group at 192 + 8h.
// Its 32 weights are runs t = tp and t = tp + 2 of 16: column 256sb + 128h + 32t + 16half + l,
// low nibble (t < 2) or high nibble (t >= 2) of low-nibble byte l, top bits 2t..2t+1 of
// high-bit byte l, scale byte 2t + half of the group.  w = d s (q - 32), summed per run as
// d s (sum q x - 32 sum x).  Even and odd superblocks go in separate steps (210 = 2 mod 4).
struct Q6_KF {
  struct Raw {
    uint32_t l[5], h[5], s[3];
    uint32_t d;
    uint32_t ph;
  };
  static __device__ __forceinline__ int steps(int cols) {
    const int nsb = cols >> 8;
    return ((nsb + 1) / 2 + 7) / 8 + (nsb / 2 + 7) / 8;
  }
  static __device__ __forceinline__ int sb_of(int cols, int step, int lane, bool& ok) {
    const int nsb = cols >> 8;
    const int se = ((nsb + 1) / 2 + 7) / 8;
    const int parity = step >= se ? 1 : 0;
    const int k = (step - parity * se) * 8 + (lane >> 3);
    const int sb = 2 * k + parity;
    ok = sb < nsb;
    return sb;
  }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    bool ok;
    const int sb = sb_of(cols, step, lane, ok);
    const int e = lane & 7, hh = e >> 2, tp = (e >> 1) & 1, half = e & 1;
    const uint8_t* A = rowp + (size_t)(ok ? sb : (sb & 1)) * 210;
    Raw r;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));  // the same for every lane of the step
    const uint8_t* B = A - r.ph;                // 4-byte aligned
    const int oL = 64 * hh + 32 * tp + 16 * half, oH = 128 + 32 * hh + 16 * half, oS = 192 + 8 * hh;
    const u32x4 a = wld16(B + oL), c = wld16(B + oH);
    r.l[0] = a.x; r.l[1] = a.y; r.l[2] = a.z; r.l[3] = a.w;
    r.h[0] = c.x; r.h[1] = c.y; r.h[2] = c.z; r.h[3] = c.w;
    const u32x2 sv = ld8(B + oS);
    r.s[0] = sv.x; r.s[1] = sv.y;
    if (r.ph != 0) {
      // the 2-byte phase needs one more dword past each piece (still inside the superblock)
      r.l[4] = wld4(B + oL + 16);
      r.h[4] = wld4(B + oH + 16);
      r.s[2] = wld4(B + oS + 8);
    } else {
      r.l[4] = r.h[4] = r.s[2] = 0;
    }
    r.d = wld2(A + 208);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane,
                                             const float* __restrict__ xl, const float* __restrict__ xs16,
                                             float (&acc)[NR]) {
    bool ok;
    const int sb = sb_of(cols, step, lane, ok);
    if (!ok) return;
    const int e = lane & 7, hh = e >> 2, tp = (e >> 1) & 1, half = e & 1;
    const int c1 = (sb << 8) + 128 * hh + 32 * tp + 16 * half;  // run t = tp; run tp + 2 is 64 columns on
    const float4* xp0 = reinterpret_cast<const float4*>(xl + xpad(c1));
    const float4* xp1 = reinterpret_cast<const float4*>(xl + xpad(c1 + 64));
    const float xs0 = xs16[c1 >> 4], xs1 = xs16[(c1 >> 4) + 4];
    const uint32_t m0f = vreg(0x0F0F0F0Fu), m30 = vreg(0x30303030u);
    const uint32_t sh0 = 4u - 2u * (uint32_t)tp;  // top bits of run tp   -> bits 4..5 (left shift)
    const uint32_t sh1 = 2u * (uint32_t)tp;       // top bits of run tp+2 -> bits 4..5 (right shift)
    float s0[NR], s1[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) s0[k] = s1[k] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 xv = xp0[i], xw = xp1[i];
#pragma unroll
      for (int k = 0; k < NR; ++k) {
        uint32_t L, H;
        if (raw[k].ph == 0) {
          L = raw[k].l[i];
          H = raw[k].h[i];
        } else {
          L = __builtin_amdgcn_alignbyte(raw[k].l[i + 1], raw[k].l[i], 2);
          H = __builtin_amdgcn_alignbyte(raw[k].h[i + 1], raw[k].h[i], 2);
        }
        // four 6-bit codes of each run, one per byte, then fp16 pairs 1024 + code
        const uint32_t c0 = and_or(H << sh0, m30, L & m0f);
        const uint32_t c1v = and_or(H >> sh1, m30, (L >> 4) & m0f);
        const uint32_t p0 = __builtin_amdgcn_perm(F16_1024, c0, PERM_B02);
        const uint32_t p1 = __builtin_amdgcn_perm(F16_1024, c0, PERM_B13);
        const uint32_t p2 = __builtin_amdgcn_perm(F16_1024, c1v, PERM_B02);
        const uint32_t p3 = __builtin_amdgcn_perm(F16_1024, c1v, PERM_B13);
        s0[k] += lo_h(p0) * xv.x;
        s0[k] += lo_h(p1) * xv.y;
        s0[k] += hi_h(p0) * xv.z;
        s0[k] += hi_h(p1) * xv.w;
        s1[k] += lo_h(p2) * xw.x;
        s1[k] += lo_h(p3) * xw.y;
        s1[k] += hi_h(p2) * xw.z;
        s1[k] += hi_h(p3) * xw.w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint32_t sb8 = 8u * (uint32_t)(2 * tp + half);  // byte of the scale in each scale dword
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      uint32_t S0, S1;
      if (raw[k].ph == 0) {
        S0 = raw[k].s[0];
        S1 = raw[k].s[1];
      } else {
        S0 = __builtin_amdgcn_alignbyte(raw[k].s[1], raw[k].s[0], 2);
        S1 = __builtin_amdgcn_alignbyte(raw[k].s[2], raw[k].s[1], 2);
      }
      const float sc0 = (float)(int8_t)((S0 >> sb8) & 0xFFu);  // run tp
      const float sc1 = (float)(int8_t)((S1 >> sb8) & 0xFFu);  // run tp + 2
      // s = sum (1024 + q) x = sum (q - 32) x + 1056 sum x
      const float tot = sc0 * (s0[k] - 1056.f * xs0) + sc1 * (s1[k] - 1056.f * xs1);
      acc[k] += h2f(raw[k].d) * tot;
    }
  }
};

// ------------------------------------------------------------------ kernel

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
// Every thread of the workgroup calls this exactly once.
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

// Greedy-pick key: larger value first, then the lower row index.
__device__ __forceinline__ unsigned long long logit_key(float v, int r) {
  v = v != v ? -INFINITY : v;  // NaN never wins
  return ((unsigned long long)order_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)r);
}

// cos and sin of the RoPE angle of pair i (0..63) of a 128-wide head at position pos: the
// angle pos * theta^(-2i/128) is formed and reduced to [-pi, pi] in fp64, then rounded.
__device__ __forceinline__ float2 rope_cs(double theta, int pos, int i) {
  const double f = pow(theta, -2.0 * (double)i / 128.0);
  double ang = (double)pos * f;
  ang -= 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  return make_float2(cs, sn);
}

template <int R, int EPI>
__device__ __forceinline__ void epilogue(const GemvArgs& a, int s, const GemvSeg& sg, int row0, int lane,
                                         const float* acc, unsigned long long& best, const float2* rope) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS) {
    if (lane < R && row0 + lane < sg.rows) {
      float v = acc[0];
#pragma unroll
      for (int k = 1; k < R; ++k) v = (lane == k) ? acc[k] : v;
      a.y[row0 + lane] = v;
    }
    if constexpr (EPI == EPI_LOGITS) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (row0 + k < sg.rows) {
          const unsigned long long key = logit_key(acc[k], row0 + k);
          best = key > best ? key : best;
        }
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
    if (lane < R / 2) {
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
          const float2 c = rope[dd >> 1];
          const float cs = c.x, sn = c.y;
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
          // V cache groups of 8 slots: [head][slot / 8][dim][slot % 8]
          uint16_t* vp = a.v_cache + (size_t)head * a.max_ctx * HD + ((size_t)(a.pos >> 3) * HD + dd) * 8 + (a.pos & 7);
          vp[0] = f2h_rne(y0);
          vp[8] = f2h_rne(y1);
        }
      }
    }
  }
}

// This wave's groups of R rows of one segment: group grp0 + k for k = wave_id, wave_id + W, ...
// over the launch's W waves.  The loads of the next step (or of the next group's first
// step) are in flight while the current step computes.  For the first segment the wave
// issues its first loads before the workgroup stages x, so that both latencies overlap;
// every wave takes part in the staging.
template <typename F, int R, int EPI>
__device__ __forceinline__ void run_segment(const GemvArgs& a, int s, int lane, int wid, int W, float* xl,
                                            float* xs16, float* red, unsigned long long& best, const float2* rope) {
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  const GemvSeg sg = a.seg[s];
  const int n_groups = (sg.rows + R - 1) / R;
  int k = (wid - sg.grp0) % W;
  if (k < 0) k += W;
  const bool any = k < n_groups;
  const int nsteps = F::steps(a.cols);

  const uint8_t* rp[NR];
  int row0 = k * R;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int r = min(row0 + j, sg.rows - 1);  // past-the-end rows re-read the last row; results dropped
    rp[j] = sg.w + (size_t)r * sg.row_bytes;
    if constexpr (EPI == EPI_SWIGLU) rp[R + j] = a.seg[1].w + (size_t)r * sg.row_bytes;
  }
  typename F::Raw cur[NR], nxt[NR];
  if (any) {
#pragma unroll
    for (int j = 0; j < NR; ++j) cur[j] = F::load(rp[j], a.cols, 0, lane);
  }
  if (s == 0) stage_x(a, xl, xs16, red);
  if (!any) return;
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
  int step = 0;
  for (;;) {
    // the next work item: the next step of these rows, or step 0 of the next group
    int nstep = step + 1, nk = k, nrow0 = row0;
    const uint8_t* nrp[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) nrp[j] = rp[j];
    if (nstep == nsteps) {
      nstep = 0;
      nk = k + W;
      nrow0 = nk * R;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int r = min(nrow0 + j, sg.rows - 1);
        nrp[j] = sg.w + (size_t)r * sg.row_bytes;
        if constexpr (EPI == EPI_SWIGLU) nrp[R + j] = a.seg[1].w + (size_t)r * sg.row_bytes;
      }
    }
    const bool more = nk < n_groups;
    if (more) {
#pragma unroll
      for (int j = 0; j < NR; ++j) nxt[j] = F::load(nrp[j], a.cols, nstep, lane);
    }
    F::template fma<NR>(cur, a.cols, step, lane, xl, xs16, acc);
    if (step == nsteps - 1) {
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]);
      epilogue<R, EPI>(a, s, sg, row0, lane, acc, best, rope);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = 0.f;
    }
    if (!more) break;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      cur[j] = nxt[j];
      rp[j] = nrp[j];
    }
    row0 = nrow0;
    k = nk;
    step = nstep;
  }
}

// At least four waves per SIMD (at most 128 VGPRs): the stream needs many waves in flight.
template <int FMTMASK, int R, int NW, int EPI>
__global__ __launch_bounds__(NW * 64, 4) void gemv_kernel(const GemvArgs a) {
  extern __shared__ float4 smem4[];
  float* xl = reinterpret_cast<float*>(smem4);
  float* xs16 = xl + xpad_len(a.cols);
  float* red = xs16 + (a.cols >> 4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wid = (int)blockIdx.x * NW + wave;
  const int W = (int)gridDim.x * NW;
  unsigned long long best = 0;
  // RoPE table for this position (visible after the barrier inside the staging of x)
  __shared__ float2 rope[64];
  if constexpr (EPI == EPI_QKV) {
    if (threadIdx.x < 64) rope[threadIdx.x] = rope_cs(a.rope_theta, a.pos, threadIdx.x);
  }
  const int nseg = (EPI == EPI_SWIGLU) ? 1 : a.nseg;
  for (int s = 0; s < nseg; ++s) {
    switch (a.seg[s].fmt) {
      case FMT_Q8_0:
        if constexpr ((FMTMASK >> FMT_Q8_0) & 1) run_segment<Q8_0F, R, EPI>(a, s, lane, wid, W, xl, xs16, red, best, rope);
        break;
      case FMT_Q4_0:
        if constexpr ((FMTMASK >> FMT_Q4_0) & 1) run_segment<Q4_0F, R, EPI>(a, s, lane, wid, W, xl, xs16, red, best, rope);
        break;
      case FMT_Q4_K:
        if constexpr ((FMTMASK >> FMT_Q4_K) & 1) run_segment<Q4_KF, R, EPI>(a, s, lane, wid, W, xl, xs16, red, best, rope);
        break;
      default:
        if constexpr ((FMTMASK >> FMT_Q6_K) & 1) run_segment<Q6_KF, R, EPI>(a, s, lane, wid, W, xl, xs16, red, best, rope);
        break;
    }
  }
  if constexpr (EPI == EPI_LOGITS) {
    // one atomic per workgroup: lane 0 of each wave holds the wave's best key
    __shared__ unsigned long long wbest[NW];
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long b = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) b = wbest[w] > b ? wbest[w] : b;
      if (b) atomicMax(a.amax, b);
    }
  }
}

// ------------------------------------------------------------------ host side

static int num_cu() {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      n_cu = n;
    else
      n_cu = 256;
  }
  return n_cu;
}

static size_t lds_for(int cols) { return sizeof(float) * (size_t)(xpad_len(cols) + (cols >> 4) + 16); }

GemvPlan gemv_plan(int epi, int cols) {
  GemvPlan p;
  p.rows_per_wave = (epi == EPI_SWIGLU) ? 1 : 2;  // the paired gate/up launch already carries two rows
  p.lds_bytes = lds_for(cols);
  // one copy of x per workgroup: when only one fits in a CU's LDS, make it 16 waves
  p.waves = p.lds_bytes > 80 * 1024 ? 16 : 8;
  return p;
}

int gemv_groups(const GemvPlan& p, int rows) { return (rows + p.rows_per_wave - 1) / p.rows_per_wave; }

template <int FMTMASK, int NW, int EPI>
static hipError_t launch_one(const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  constexpr int R = (EPI == EPI_SWIGLU) ? 1 : 2;
  auto kern = gemv_kernel<FMTMASK, R, NW, EPI>;
  // resident workgroups per CU at this LDS size, cached per instantiation
  static int per_cu = 0;
  static size_t per_cu_lds = 0;
  if (per_cu == 0 || per_cu_lds != plan.lds_bytes) {
    // the dynamic LDS this launch needs (static LDS of the kernel comes on top)
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)plan.lds_bytes);
    if (e != hipSuccess) return e;
    int n = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NW * 64, plan.lds_bytes);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
    if (NT_GEMV_WG_PER_CU_MAX > 0 && per_cu > NT_GEMV_WG_PER_CU_MAX) per_cu = NT_GEMV_WG_PER_CU_MAX;
    per_cu_lds = plan.lds_bytes;
  }
  // as many resident waves as the chip holds, but no idle workgroups
  const int grid = max(1, min((n_groups + NW - 1) / NW, per_cu * num_cu()));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), plan.lds_bytes, s, a);
  return hipGetLastError();
}

template <int FMTMASK, int EPI>
static hipError_t launch_nw(const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  switch (plan.waves) {
    case 8: return launch_one<FMTMASK, 8, EPI>(plan, n_groups, a, s);
    case 16: return launch_one<FMTMASK, 16, EPI>(plan, n_groups, a, s);
    default: return hipErrorInvalidConfiguration;
  }
}

template <int EPI>
static hipError_t launch_mask(int fmt_mask, const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  switch (fmt_mask) {
    case 1 << FMT_Q8_0: return launch_nw<1 << FMT_Q8_0, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q4_0: return launch_nw<1 << FMT_Q4_0, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q4_K: return launch_nw<1 << FMT_Q4_K, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q6_K: return launch_nw<1 << FMT_Q6_K, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q4_K) | (1 << FMT_Q6_K): return launch_nw<(1 << FMT_Q4_K) | (1 << FMT_Q6_K), EPI>(plan, n_groups, a, s);
    default: return launch_nw<15, EPI>(plan, n_groups, a, s);
  }
}

hipError_t gemv_launch(int fmt_mask, int epi, const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_mask<EPI_STORE>(fmt_mask, plan, n_groups, a, s);
    case EPI_RESID: return launch_mask<EPI_RESID>(fmt_mask, plan, n_groups, a, s);
    case EPI_SWIGLU: return launch_mask<EPI_SWIGLU>(fmt_mask, plan, n_groups, a, s);
    case EPI_QKV: return launch_mask<EPI_QKV>(fmt_mask, plan, n_groups, a, s);
    default: return launch_mask<EPI_LOGITS>(fmt_mask, plan, n_groups, a, s);
  }
}

}  // namespace nt
