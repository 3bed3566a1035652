// Fused dequantize-and-GEMV over GGML-style block-quantized weights, batch 1, gfx950.
//
// The decode path reads every weight once per token (70B PCIe P2P article,
// blog.hotdry.top, §传统数据路径的性能瓶颈分析), so these kernels are an HBM stream with a
// tight ALU budget.  Two paths:
//  * register path (gemv_kernel): persistent workgroups, as many as stay resident; each
//    stages the activation vector x (optionally RMS-normalised on the way in) into LDS
//    once, as signed 8-bit limbs with a power-of-two scale per 32 columns and exact fp32
//    sums per 16 columns; the work is groups of R rows (a gate/up row pair for the SwiGLU
//    launch) dealt round-robin to every wave; a wave walks its rows' blocks in steps, a
//    lane taking one fixed slice of a block (a Q8_0/Q4_0 block, a quarter of a
//    Q4_K/Q5_K superblock, an eighth of a Q6_K one) with 128-bit loads, the loads of the
//    next step in flight while the current one computes;
//  * streamed path (gemv_stream_kernel, Q6_K and the 32-weight formats): waves split the
//    columns into slices, hold their x slice in registers and stream their rows' bytes
//    HBM -> LDS with global->LDS transfers.
// Codes become bytes (nibble masks; high bits rotated into place) and meet the limbs in
// v_dot4_i32_i8, four exact 8-bit products per instruction; each 16- or 32-column integer
// sum is scaled once; offsets and mins use the fp32 x sums.  Blocks of 34, 18 and 210
// bytes sit at 2-byte phases, realigned with v_alignbyte.  Epilogues fuse the residual
// add, SwiGLU, RoPE + fp16 KV append, or the greedy argmax.
// No matrix cores in the GEMVs: at batch 1 this is not a dense contraction (the k-token GEMM
// below uses them for Q4_K, Q5_K and Q6_K at 3 to 8 tokens, where it is one).
#include <atomic>
#include <type_traits>

#include "common.h"
#include "gemv.h"

namespace nt {

// ------------------------------------------------------------------ helpers



// Launch-geometry and load-policy defaults (overridable at build time).
#ifndef NT_GEMV_WG_PER_CU_MAX
#define NT_GEMV_WG_PER_CU_MAX 0  // 0: as many workgroups per CU as stay resident
#endif
#ifndef NT_GEMV_NONTEMPORAL
#define NT_GEMV_NONTEMPORAL 0
#endif
#ifndef NT_GEMV_ROWS
#define NT_GEMV_ROWS 2  // rows per work item of the register path (the gate/up pair always takes 1 of each)
#endif
#ifndef NT_GEMV_DEPTH
#define NT_GEMV_DEPTH 2  // work items in flight per wave on the register path (gate/up pair: 2)
#endif
#ifndef NT_GEMV_DEPTH_PAIR
#define NT_GEMV_DEPTH_PAIR 2  // the same for the gate/up pair
#endif
#ifndef NT_GEMV_DEPTH_QKV
#define NT_GEMV_DEPTH_QKV 2  // the same for the q/k/v launch
#endif
#ifndef NT_GEMV_STREAM
#define NT_GEMV_STREAM 1  // the streamed (global->LDS) path wherever the shape allows it
#endif

// Weight loads, through global-address-space pointers: a load the compiler can only prove
// to be generic becomes a flat load, which also counts against the LDS wait counter, so every
// wait for an LDS read would wait for the prefetched weights too.  Nontemporal loads were
// measured slower for these (20-45%: a lane's line is read by two instructions), so plain
// cached loads are the default here; the streamed path's whole-line transfers do use them.
#define NT_GPTR(T, p) ((const __attribute__((address_space(1))) T*)(p))
#if NT_GEMV_NONTEMPORAL
__device__ __forceinline__ u32x4 wld16(const uint8_t* p) { return __builtin_nontemporal_load(NT_GPTR(u32x4, p)); }
__device__ __forceinline__ uint32_t wld4(const uint8_t* p) { return __builtin_nontemporal_load(NT_GPTR(uint32_t, p)); }
__device__ __forceinline__ uint32_t wld2(const uint8_t* p) { return __builtin_nontemporal_load(NT_GPTR(uint16_t, p)); }
#else
__device__ __forceinline__ u32x4 wld16(const uint8_t* p) { return *NT_GPTR(u32x4, p); }
__device__ __forceinline__ uint32_t wld4(const uint8_t* p) { return *NT_GPTR(uint32_t, p); }
__device__ __forceinline__ uint32_t wld2(const uint8_t* p) { return *NT_GPTR(uint16_t, p); }
#endif
__device__ __forceinline__ u32x2 wld8(const uint8_t* p) { return *NT_GPTR(u32x2, p); }

typedef uint32_t u32x4a16 __attribute__((ext_vector_type(4), aligned(16)));

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

// ------------------------------------------------------------------ activations as limbs
//
// The register path keeps x in LDS as XL signed 8-bit limbs per column.  Each block of 32
// columns has a power-of-two scale s, the smallest with max |x| / s <= 127, and the
// fixed-point value X = rint(x / s 256^(XL-1)) is split into balanced base-256 digits:
//   X = 256^(XL-1) x1 + ... + x_XL,   x1 in [-127, 127], the others in [-128, 127],
// so x is represented to within s 2^-(8 XL - 7) < max |x of the block| 2 / (127 2^(8 XL - 7)):
// / 8.3e6 with three limbs, / 32512 with two.  Every step is exact in fp32 (scaling by a
// power of two, rounding to an integer below 2^24).  Three limbs are the default: with two,
// a block holding one activation 10^4 times its neighbours (as large outlier channels do)
// leaves some rows within a few times of a 1e-3 sum |w x| error; with three, within 1e-6.  The weight codes are small integers, so over a run of columns
// sum q x = s (D1 + D2 / 256 + D3 / 65536) where Dk = sum q xk is formed exactly by
// v_dot4_i32_i8 (four 8-bit products and the accumulation in one instruction), in place of
// a convert and an fp32 FMA per weight.  The offset and min terms of the formats use exact
// fp32 sums of x per 16 columns.
// A limb plane holds byte c at xq_off(c): 16 pad bytes after every 64 columns, so lanes that
// read 16-column runs 64 columns apart with 128-bit reads spread over the banks.
#ifndef NT_GEMV_XLIMBS
#define NT_GEMV_XLIMBS 3
#endif
constexpr int XL = NT_GEMV_XLIMBS;
static_assert(XL == 2 || XL == 3, "two or three limbs");

__host__ __device__ __forceinline__ int xq_off(int c) { return c + ((c >> 6) << 4); }
__host__ __device__ __forceinline__ int xq_plane(int cols) { return (xq_off(cols) + 15) & ~15; }
// LDS bytes of one token's staged chunk in the k-token GEMM: limb planes, a scale per 32
// columns and a sum per 16, rounded to 16 bytes
// (fp32 x instead of the limb planes for the unquantized formats, f)
__host__ __device__ __forceinline__ size_t gemm_lds_per_token(int cols, bool f = false) {
  return ((f ? sizeof(float) * (size_t)cols : (size_t)XL * xq_plane(cols)) +
          sizeof(float) * (size_t)((cols >> 5) + (cols >> 4)) + 15) & ~(size_t)15;
}

// The staged activation vector, as the register-path kernels see it in LDS.
struct XLimbs {
  uint8_t* q = nullptr;   // XL planes of xq_plane(cols) bytes (null: not staged, no quantized format in the launch)
  int plane = 0;
  float* sc = nullptr;    // scale s / 256^(XL-1) per 32 columns
  float* s16 = nullptr;   // sum of x per 16 columns (fp32)
  float* xf = nullptr;    // x itself, fp32, for the unquantized formats (null: not staged)
};

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}
// The same with c = 0, in the three-operand encoding with an inline-constant 0: the compiler
// otherwise picks the accumulating two-operand form and zeroes the destination first, one
// extra instruction per run of products.
__device__ __forceinline__ int sdot4_0(uint32_t a, uint32_t b) {
  int r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// 256^(XL-1) (D1 + D2 / 256 (+ D3 / 65536)): the staged scale per 32 columns is stored as
// s / 256^(XL-1), so that the product of the two is s (D1 + ...).  |Dk| < 2^20 here (at most
// 32 codes of magnitude <= 128 times digits of magnitude <= 128), so 256 D1 + D2 fits an int.
__device__ __forceinline__ float limb_sum(const int (&d)[XL]) {
  if constexpr (XL == 3)
    return (float)d[0] * 65536.f + (float)((d[1] << 8) + d[2]);
  else
    return (float)((d[0] << 8) + d[1]);
}
// The fp32 sums of the four 16-column runs from c (a multiple of 64) in one 16-byte read.
// A lane reading them as two pairs of dwords 16 bytes from its neighbour's made each dword
// access a four-way LDS bank conflict; the 16-byte read is conflict-free.  The sums start on
// a 16-byte boundary whenever the columns are whole 256-column superblocks (cols / 32
// scales of 4 bytes before them, after 16-byte-aligned limb planes), as for Q4_K and Q5_K.
__device__ __forceinline__ float4 s16x4(const XLimbs& xs, int c) {
  return *reinterpret_cast<const float4*>(xs.s16 + (c >> 4));
}
// The limbs of 16 columns starting at c (a multiple of 16): 4 dwords per plane.
struct XRun {
  u32x4 p[XL];
};
__device__ __forceinline__ XRun x_run(const XLimbs& xs, int c) {
  XRun r;
  const uint8_t* b = xs.q + xq_off(c);
#pragma unroll
  for (int k = 0; k < XL; ++k) {
    const u32x4a16 v = *reinterpret_cast<const u32x4a16*>(b + k * xs.plane);
    r.p[k] = u32x4{v.x, v.y, v.z, v.w};
  }
  return r;
}
// d[l] += sum over the four bytes of q and of dword i of limb plane l (first: d[l] = that sum,
// so that the first product of a run takes an immediate 0 instead of a zeroed register)
__device__ __forceinline__ void dot_limbs(uint32_t q, const XRun& x, int i, int (&d)[XL], bool first = false) {
#pragma unroll
  for (int l = 0; l < XL; ++l) d[l] = first ? sdot4_0(q, x.p[l][i]) : sdot4(q, x.p[l][i], d[l]);
}
template <int NR>
__device__ __forceinline__ void zero_limbs(int (&d)[NR][XL]) {
#pragma unroll
  for (int k = 0; k < NR; ++k)
#pragma unroll
    for (int l = 0; l < XL; ++l) d[k][l] = 0;
}

// t[k] = (sum over 16 columns at c of code k times x~) / s, for NR rows of 16 codes (4 dwords)
// each: the limb planes are read one at a time, each feeding every row
template <int NR>
__device__ __forceinline__ void run_dot(const XLimbs& xs, int c, const uint32_t (&q)[NR][4], float (&t)[NR]) {
  int d[NR][XL];
  const uint8_t* b = xs.q + xq_off(c);
#pragma unroll
  for (int l = 0; l < XL; ++l) {
    const u32x4a16 x = *reinterpret_cast<const u32x4a16*>(b + l * xs.plane);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      d[k][l] = sdot4(q[k][0], x.x, 0);
      d[k][l] = sdot4(q[k][1], x.y, d[k][l]);
      d[k][l] = sdot4(q[k][2], x.z, d[k][l]);
      d[k][l] = sdot4(q[k][3], x.w, d[k][l]);
    }
  }
#pragma unroll
  for (int k = 0; k < NR; ++k) t[k] = limb_sum(d[k]);
}

// ------------------------------------------------------------------ formats
//
// Each format provides:
//   Raw                          registers of one row's slice for one step
//   steps(cols)                  steps per row
//   load(rowp, cols, step, lane) issue the global loads of one row's slice
//   fma(raw[NR], ..., acc[NR])   consume them: acc[k] += this step's part of row k

// Q8_0: lane = one 34-byte block; steps visit the even blocks, then the odd ones.
struct Q8_0F {
  // the block's 34 bytes from the dword boundary B at or before it: phase 0 (block at B):
  // w = bytes 0..31, e = bytes 32..33; phase 2 (block at B + 2): e = the scale (bytes 2..3),
  // w = bytes 4..35.  The same three loads either way, so the count in flight is static.
  struct Raw {
    uint32_t w[8];
    uint32_t e;
    uint32_t ph;
  };
  static __host__ __device__ __forceinline__ int steps(int cols) {
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
    const uint8_t* A = rowp + (uint32_t)(ok ? blk : (blk & 1)) * 34u;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));  // the same for every lane of the step
    const uint8_t* B = A - r.ph;
    const int o = r.ph ? 4 : 0;
    const u32x4 a = wld16(B + o), b = wld16(B + o + 16);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    r.e = wld2(r.ph ? A : B + 32);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    bool ok;
    const int blk = block_of(cols, step, lane, ok);
    if (!ok) return;
    uint32_t q[NR][8];
    float d[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (raw[k].ph == 0) {
        d[k] = h2f(raw[k].w[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = __builtin_amdgcn_alignbyte(i < 7 ? raw[k].w[i + 1] : raw[k].e, raw[k].w[i], 2);
      } else {
        d[k] = h2f(raw[k].e);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[k][i] = raw[k].w[i];
      }
    }
    apply<NR>(q, d, blk, xs, acc);
  }
  // acc[k] += d[k] s sum_i q[k][i] x~_i over block blk (32 int8 codes in 8 dwords)
  template <int NR>
  static __device__ __forceinline__ void apply(const uint32_t (&q)[NR][8], const float (&d)[NR], int blk,
                                               const XLimbs& xs, float (&acc)[NR]) {
    int D[NR][XL];
    zero_limbs(D);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const XRun x = x_run(xs, (blk << 5) + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NR; ++k) dot_limbs(q[k][4 * h + i], x, i, D[k], h == 0 && i == 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float s = xs.sc[blk];
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] += (d[k] * s) * limb_sum(D[k]);
  }
};

// Q8_0T: Q8_0 in tiles of 64 blocks (common.h); lane l takes block l of a tile, a step is one
// tile, and the two 16-byte code loads and the 2-byte scale load of a wave each read whole
// lines (1 KiB, 1 KiB, 128 B), with the nontemporal policy for launches of at least 10^8
// weights (NTL) as for Q4_KT; the products are Q8_0F's.
template <bool NTL>
struct Q8_0TF {
  struct Raw {
    uint32_t w[8];
    uint32_t e;
  };
  static __host__ __device__ __forceinline__ int steps(int cols) { return ((cols >> 5) + 63) / 64; }
  static __device__ __forceinline__ u32x4 ld(const uint8_t* p) {
    if constexpr (NTL) return __builtin_nontemporal_load(NT_GPTR(u32x4, p));
    else return *NT_GPTR(u32x4, p);
  }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    const int nb = cols >> 5;
    int b = step * 64 + lane;
    b = b < nb ? b : 0;
    const u32x4 a = ld(rowp + q8t_qa(nb, b)), c = ld(rowp + q8t_qb(nb, b));
    Raw r;
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = c.x; r.w[5] = c.y; r.w[6] = c.z; r.w[7] = c.w;
    if constexpr (NTL) r.e = __builtin_nontemporal_load(NT_GPTR(uint16_t, rowp + q8t_d(nb, b)));
    else r.e = *NT_GPTR(uint16_t, rowp + q8t_d(nb, b));
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    const int blk = step * 64 + lane;
    if (blk >= (cols >> 5)) return;
    uint32_t q[NR][8];
    float d[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      d[k] = h2f(raw[k].e);
#pragma unroll
      for (int i = 0; i < 8; ++i) q[k][i] = raw[k].w[i];
    }
    Q8_0F::apply<NR>(q, d, blk, xs, acc);
  }
};

// Q4_0: lane = one 18-byte block; weights 0..15 are the low nibbles, 16..31 the high ones.
// w = d (q - 8): summed as d (s sum q x~ - 8 sum x).
struct Q4_0F {
  // phase 0 (block at the dword boundary B): w = bytes 0..15, e = bytes 16..17; phase 2:
  // e = the scale (bytes 2..3), w = bytes 4..19 (as for Q8_0: two loads either way)
  struct Raw {
    uint32_t w[4];
    uint32_t e;
    uint32_t ph;
  };
  static __device__ __forceinline__ int steps(int cols) { return Q8_0F::steps(cols); }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    bool ok;
    const int blk = Q8_0F::block_of(cols, step, lane, ok);
    Raw r;
    const uint8_t* A = rowp + (uint32_t)(ok ? blk : (blk & 1)) * 18u;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));
    const uint8_t* B = A - r.ph;
    const u32x4 a = wld16(B + (r.ph ? 4 : 0));
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.e = wld2(r.ph ? A : B + 16);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    bool ok;
    const int blk = Q8_0F::block_of(cols, step, lane, ok);
    if (!ok) return;
    uint32_t q[NR][4];
    float d[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (raw[k].ph == 0) {
        d[k] = h2f(raw[k].w[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[k][i] = __builtin_amdgcn_alignbyte(i < 3 ? raw[k].w[i + 1] : raw[k].e, raw[k].w[i], 2);
      } else {
        d[k] = h2f(raw[k].e);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[k][i] = raw[k].w[i];
      }
    }
    const uint32_t m0f = vreg(0x0F0F0F0Fu);
    int D[NR][XL];
    zero_limbs(D);
    // h = 0: low nibbles, columns 0..15 of the block; h = 1: high nibbles, columns 16..31
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const XRun x = x_run(xs, (blk << 5) + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NR; ++k)
          dot_limbs(h == 0 ? (q[k][i] & m0f) : ((q[k][i] >> 4) & m0f), x, i, D[k], h == 0 && i == 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float s = xs.sc[blk];
    const float xsum = xs.s16[2 * blk] + xs.s16[2 * blk + 1];
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] += d[k] * (s * limb_sum(D[k]) - 8.f * xsum);
  }
};

// Q4_K: lane = quarter g of a 144-byte superblock: the 32 nibble bytes at 16 + 32 g, whose
// low nibbles are sub-block 2g and high nibbles sub-block 2g+1 (64 weights); 16 superblocks
// per step.  w = d sc q - dmin m, summed per sub-block as d sc s (sum q x~) - dmin m (sum x);
// a sub-block is one 32-column scale block of x.
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
    // a 32-bit offset from the row's (wave-uniform) start: the loads take the scalar base and
    // a vector offset, with no 64-bit address arithmetic per lane
    const uint32_t off = (uint32_t)sb * 144u;
    Raw r;
    r.hd = wld16(rowp + off);
    r.qa = wld16(rowp + (off + 16u + 32u * (uint32_t)g));
    r.qb = wld16(rowp + (off + 32u + 32u * (uint32_t)g));
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    const int nsb = cols >> 8;
    const int sb = step * 16 + (lane >> 2);
    if (sb >= nsb) return;
    const int g = lane & 3;
    const int c0 = (sb << 8) + (g << 6);
    const uint32_t m0f = vreg(0x0F0F0F0Fu), mf0 = 0xF0F0F0F0u, m80 = 0x80808080u;
    int da[NR][XL], db[NR][XL];
    zero_limbs(da);
    zero_limbs(db);
    // run h of 16 columns at c0 + 16 h: low nibbles of qa (h = 0) and qb (h = 1) belong to
    // sub-block 2g, high nibbles of qa (h = 2) and qb (h = 3) to sub-block 2g + 1.  A high
    // nibble n is used in place, as the signed byte (16 n) ^ 0x80 = 16 n - 128 (one
    // three-input bit operation instead of a shift and a mask), so db holds 16 (sum n X) -
    // 128 (sum X) over the sub-block; the 128 (sum X) part is restored from the fp32 sum of
    // x below.
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const XRun x = x_run(xs, c0 + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const uint32_t v = (h & 1) ? raw[k].qb[i] : raw[k].qa[i];
          if (h < 2)
            dot_limbs(v & m0f, x, i, da[k], h == 0 && i == 0);
          else
            dot_limbs((v & mf0) ^ m80, x, i, db[k], h == 2 && i == 0);
        }
      // keep each run's LDS reads next to their use
      __builtin_amdgcn_sched_barrier(0);
    }
    const float sA = xs.sc[c0 >> 5], sB = xs.sc[(c0 >> 5) + 1];
    const float4 x4 = s16x4(xs, c0);
    const float xa = x4.x + x4.y, xb = x4.z + x4.w;
    const float sB16 = sB * 0.0625f, xb8 = 8.f * xb;
    // 6-bit scales and mins of sub-blocks 2g, 2g+1 gathered as the bytes [sc_a, sc_b, m_a, m_b]
    // from the scale words Y (bytes 4..7), Z (8..11), W (12..15), p = 2 (g & 1):
    //  sub-blocks 0..3: scale = bits 0..5 of Y byte p (+1), min = bits 0..5 of Z byte p (+1);
    //  sub-blocks 4..7: low four bits from W byte p (+1) (scale: low nibble, min: high
    //  nibble), top two bits from bits 6..7 of Y (scale) and Z (min) byte p (+1).
    const uint32_t p = 2u * (uint32_t)(g & 1);
    const uint32_t sel = p | ((p + 1) << 8) | ((p + 4) << 16) | ((p + 5) << 24);  // [Y p, Y p+1, Z p, Z p+1]
    const bool upper = g >= 2;
    const uint32_t mlow = vreg(upper ? 0x0F0F0F0Fu : 0x3F3F3F3Fu), mtop = vreg(upper ? 0x30303030u : 0u);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint32_t Y = raw[k].hd.y, Z = raw[k].hd.z, W = raw[k].hd.w;
      const uint32_t yz = __builtin_amdgcn_perm(Z, Y, sel);
      const uint32_t lo = upper ? __builtin_amdgcn_perm(W >> 4, W, sel) : yz;  // [W p, W p+1, W p>>4, W p+1>>4]
      const uint32_t sm = and_or(yz >> 2, mtop, lo & mlow);
      const float d = h2f(raw[k].hd.x), dmin = h2f(raw[k].hd.x >> 16);
      // sub-block 2g + 1: sB (sum n X) = (sB / 16) db + 8 sB (sum X), and sB (sum X) is the
      // sum of the staged x, within rounding of the fp32 sum xb
      const float sb = d * ub1(sm);
      acc[k] += (d * sA * ub0(sm)) * limb_sum(da[k]);
      acc[k] += (sb * sB16) * limb_sum(db[k]);
      acc[k] += sb * xb8;
      acc[k] -= dmin * (ub2(sm) * xa + ub3(sm) * xb);
    }
  }
};

// Q4_KT: Q4_K in tiles of 16 superblocks (common.h), the same lane work as Q4_KF; a step is
// one tile, and each of the three 16-byte loads of a wave reads whole lines (the headers,
// four lanes to an address, then 1 KiB of code bytes twice).  NTL: the nontemporal policy,
// which the large launches take: with GGUF's layout a lane's line is split between two load
// instructions and the policy costs 20-45%, while on whole lines it lifts the read rate
// (measured, 70B decode, Q4_K -> Q4_KT: gate/up pair 50.0 -> 46.2 us, LM head 106 -> 96.3 us);
// the small launches keep cached loads (q/k/v 19.4 against 20.3 us with the policy, O 13.4
// against 13.7 us; 21.0 and 13.6 us in Q4_K's block order).
__device__ __forceinline__ u32x4 wld16nt(const uint8_t* p) { return __builtin_nontemporal_load(NT_GPTR(u32x4, p)); }

template <bool NTL>
struct Q4_KTF : Q4_KF {
  static __device__ __forceinline__ u32x4 ld(const uint8_t* p) {
    if constexpr (NTL) return wld16nt(p);
    else return *NT_GPTR(u32x4, p);
  }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    const int nsb = cols >> 8;
    int sb = step * 16 + (lane >> 2);
    sb = sb < nsb ? sb : 0;
    const int g = lane & 3;
    Raw r;
    r.hd = ld(rowp + q4kt_head(nsb, sb));
    r.qa = ld(rowp + q4kt_qa(nsb, sb, g));
    r.qb = ld(rowp + q4kt_qb(nsb, sb, g));
    return r;
  }
};

// Q5_K: the Q4_K lane layout over a 176-byte superblock (16-byte aligned: no phases), with
// a fifth code bit worth 16: column l (0..31) of sub-block j has it in bit j of high-bit byte
// l (bytes 16..47, which all four lanes of the superblock read).  Run h of the quarter takes
// high-bit bytes 16 (h & 1) .. +15 and bit 2g + (h >> 1); the nibbles sit at 48 + 32 g.
// The bit is rotated into bit 4 of each byte and OR-ed onto the nibble: codes 0..31.
struct Q5_KF {
  struct Raw {
    u32x4 hd, ha, hb, qa, qb;
  };
  static __device__ __forceinline__ int steps(int cols) { return ((cols >> 8) + 15) / 16; }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    const int nsb = cols >> 8;
    int sb = step * 16 + (lane >> 2);
    sb = sb < nsb ? sb : 0;
    const int g = lane & 3;
    const uint8_t* p = rowp + (uint32_t)sb * 176u;
    Raw r;
    r.hd = wld16(p);
    r.ha = wld16(p + 16);
    r.hb = wld16(p + 32);
    r.qa = wld16(p + 48 + 32 * g);
    r.qb = wld16(p + 64 + 32 * g);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    const int nsb = cols >> 8;
    const int sb = step * 16 + (lane >> 2);
    if (sb >= nsb) return;
    const int g = lane & 3;
    const int c0 = (sb << 8) + (g << 6);
    const uint32_t m0f = vreg(0x0F0F0F0Fu), m10 = vreg(0x10101010u);
    // rotations that bring bit 2g (runs 0, 1) and bit 2g + 1 (runs 2, 3) of each byte to bit 4
    const uint32_t rot_a = (uint32_t)(2 * g + 28) & 31u, rot_b = (uint32_t)(2 * g + 29) & 31u;
    int da[NR][XL], db[NR][XL];
    zero_limbs(da);
    zero_limbs(db);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const XRun x = x_run(xs, c0 + 16 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const uint32_t v = (h & 1) ? raw[k].qb[i] : raw[k].qa[i];
          const uint32_t hv = (h & 1) ? raw[k].hb[i] : raw[k].ha[i];
          if (h < 2)
            dot_limbs(and_or(__builtin_amdgcn_alignbit(hv, hv, rot_a), m10, v & m0f), x, i, da[k], h == 0 && i == 0);
          else
            dot_limbs(and_or(__builtin_amdgcn_alignbit(hv, hv, rot_b), m10, (v >> 4) & m0f), x, i, db[k],
                      h == 2 && i == 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float sA = xs.sc[c0 >> 5], sB = xs.sc[(c0 >> 5) + 1];
    const float4 x4 = s16x4(xs, c0);
    const float xa = x4.x + x4.y, xb = x4.z + x4.w;
    // scales and mins exactly as Q4_K's (same 12-byte packing at bytes 4..15)
    const uint32_t p = 2u * (uint32_t)(g & 1);
    const uint32_t sel = p | ((p + 1) << 8) | ((p + 4) << 16) | ((p + 5) << 24);
    const bool upper = g >= 2;
    const uint32_t mlow = vreg(upper ? 0x0F0F0F0Fu : 0x3F3F3F3Fu), mtop = vreg(upper ? 0x30303030u : 0u);
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const uint32_t Y = raw[k].hd.y, Z = raw[k].hd.z, W = raw[k].hd.w;
      const uint32_t yz = __builtin_amdgcn_perm(Z, Y, sel);
      const uint32_t lo = upper ? __builtin_amdgcn_perm(W >> 4, W, sel) : yz;
      const uint32_t sm = and_or(yz >> 2, mtop, lo & mlow);
      const float d = h2f(raw[k].hd.x), dmin = h2f(raw[k].hd.x >> 16);
      acc[k] += (d * sA * ub0(sm)) * limb_sum(da[k]);
      acc[k] += (d * sB * ub1(sm)) * limb_sum(db[k]);
      acc[k] -= dmin * (ub2(sm) * xa + ub3(sm) * xb);
    }
  }
};

// Q5_KT: Q5_K in tiles of 16 superblocks (common.h), the same lane work as Q5_KF, each of its
// five loads reading whole lines (the headers and high bits four lanes to an address); the
// nontemporal policy from 10^8 weights as for Q4_KT.
template <bool NTL>
struct Q5_KTF : Q5_KF {
  static __device__ __forceinline__ u32x4 ld(const uint8_t* p) {
    if constexpr (NTL) return __builtin_nontemporal_load(NT_GPTR(u32x4, p));
    else return *NT_GPTR(u32x4, p);
  }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    const int nsb = cols >> 8;
    int sb = step * 16 + (lane >> 2);
    sb = sb < nsb ? sb : 0;
    const int g = lane & 3;
    Raw r;
    r.hd = ld(rowp + q5kt_hd(nsb, sb));
    r.ha = ld(rowp + q5kt_ha(nsb, sb));
    r.hb = ld(rowp + q5kt_hb(nsb, sb));
    r.qa = ld(rowp + q5kt_qa(nsb, sb, g));
    r.qb = ld(rowp + q5kt_qb(nsb, sb, g));
    return r;
  }
};

// Q6_K: lane = one eighth of a 210-byte superblock, (h, tp, half) with h, tp, half in {0,1}:
// the 16 low-nibble bytes at 64h + 32tp + 16half (the next eight lanes read the next 128
// bytes), the 16 high-bit bytes at 128 + 32h + 16half, and the scale group at 192 + 8h.
// Its 32 weights are runs t = tp and t = tp + 2 of 16: column 256sb + 128h + 32t + 16half + l,
// low nibble (t < 2) or high nibble (t >= 2) of low-nibble byte l, top bits 2t..2t+1 of
// high-bit byte l, scale byte 2t + half of the group.  w = d sc (q - 32), summed per run as
// d sc (s sum q x~ - 32 sum x).  Even and odd superblocks go in separate steps (210 = 2 mod 4).
struct Q6_KF {
  struct Raw {
    uint32_t l[5], h[5], s[3];
    uint32_t d;
    uint32_t ph;
  };
  static __host__ __device__ __forceinline__ int steps(int cols) {
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
    const uint8_t* A = rowp + (uint32_t)(ok ? sb : (sb & 1)) * 210u;
    Raw r;
    r.ph = uni((uint32_t)((uintptr_t)A & 3u));  // the same for every lane of the step
    const uint8_t* B = A - r.ph;                // 4-byte aligned
    const int oL = 64 * hh + 32 * tp + 16 * half, oH = 128 + 32 * hh + 16 * half, oS = 192 + 8 * hh;
    const u32x4 a = wld16(B + oL), c = wld16(B + oH);
    r.l[0] = a.x; r.l[1] = a.y; r.l[2] = a.z; r.l[3] = a.w;
    r.h[0] = c.x; r.h[1] = c.y; r.h[2] = c.z; r.h[3] = c.w;
    const u32x2 sv = wld8(B + oS);
    r.s[0] = sv.x; r.s[1] = sv.y;
    // the 2-byte phase needs one more dword past each piece (inside the superblock); the
    // loads are issued at either phase so that the count in flight is static (at phase 0
    // the scale dword re-reads an earlier one: bytes 208..211 would run past the block)
    r.l[4] = wld4(B + oL + 16);
    r.h[4] = wld4(B + oH + 16);
    r.s[2] = wld4(B + oS + (r.ph ? 8 : 4));
    r.d = wld2(A + 208);
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
    bool ok;
    const int sb = sb_of(cols, step, lane, ok);
    if (!ok) return;
    const int e = lane & 7, hh = e >> 2, tp = (e >> 1) & 1, half = e & 1;
    const int c1 = (sb << 8) + 128 * hh + 32 * tp + 16 * half;  // run t = tp; run tp + 2 is 64 columns on
    const uint32_t m0f = vreg(0x0F0F0F0Fu), m30 = vreg(0x30303030u);
    const uint32_t sh0 = 4u - 2u * (uint32_t)tp;  // top bits of run tp   -> bits 4..5 (left shift)
    const uint32_t sh1 = 2u * (uint32_t)tp;       // top bits of run tp+2 -> bits 4..5 (right shift)
    // four 6-bit codes per dword, one per byte: cA of run tp, cB of run tp + 2
    uint32_t cA[NR][4], cB[NR][4];
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t L, H;
        if (raw[k].ph == 0) {
          L = raw[k].l[i];
          H = raw[k].h[i];
        } else {
          L = __builtin_amdgcn_alignbyte(raw[k].l[i + 1], raw[k].l[i], 2);
          H = __builtin_amdgcn_alignbyte(raw[k].h[i + 1], raw[k].h[i], 2);
        }
        cA[k][i] = and_or(H << sh0, m30, L & m0f);
        cB[k][i] = and_or(H >> sh1, m30, (L >> 4) & m0f);
      }
    float tA[NR], tB[NR];
    run_dot(xs, c1, cA, tA);
    run_dot(xs, c1 + 64, cB, tB);
    const float s0 = xs.sc[c1 >> 5], s1 = xs.sc[(c1 + 64) >> 5];
    const float xs0 = xs.s16[c1 >> 4], xs1 = xs.s16[(c1 >> 4) + 4];
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
      const float tot = sc0 * (s0 * tA[k] - 32.f * xs0) + sc1 * (s1 * tB[k] - 32.f * xs1);
      acc[k] += h2f(raw[k].d) * tot;
    }
  }
};

// F16 / F32: unquantized rows (GGUF's F16 and F32 tensors).  Lane = 16 consecutive bytes per
// load, four loads per step at 1 KiB apart, so each load instruction reads 1 KiB of the row:
// F16 columns 2048 step + 512 i + 8 lane .. +7, F32 columns 1024 step + 256 i + 4 lane .. +3.
// The products are fp32 FMAs against the fp32 copy of x (w is exact in fp32).  Columns are a
// multiple of 32, so a load is wholly inside or wholly past the row.
template <bool H>
struct FloatF {
  static constexpr int CPL = H ? 8 : 4;  // columns per 16-byte load
  static constexpr int SHIFT = H ? 11 : 10;  // log2 of the columns of a step
  struct Raw {
    u32x4 v[4];
  };
  static __device__ __forceinline__ int col(int step, int i, int lane) {
    return (step << SHIFT) + i * 64 * CPL + lane * CPL;
  }
  static __device__ __forceinline__ int steps(int cols) { return (cols + (1 << SHIFT) - 1) >> SHIFT; }
  static __device__ __forceinline__ Raw load(const uint8_t* rowp, int cols, int step, int lane) {
    Raw r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = col(step, i, lane);
      c = c < cols ? c : 0;  // past the row end: reread its start (dropped)
      r.v[i] = wld16(rowp + (uint32_t)c * (H ? 2u : 4u));
    }
    return r;
  }
  template <int NR>
  static __device__ __forceinline__ void fma(const Raw (&raw)[NR], int cols, int step, int lane, const XLimbs& xs,
                                             float (&acc)[NR]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = col(step, i, lane);
      if (c >= cols) break;  // the later loads of the step are past the end too
      if constexpr (H) {
        const float4 x0 = *reinterpret_cast<const float4*>(xs.xf + c);
        const float4 x1 = *reinterpret_cast<const float4*>(xs.xf + c + 4);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const u32x4 w = raw[k].v[i];
          float t0 = h2f(w.x) * x0.x, t1 = h2f(w.x >> 16) * x0.y;
          t0 = fmaf(h2f(w.y), x0.z, t0); t1 = fmaf(h2f(w.y >> 16), x0.w, t1);
          t0 = fmaf(h2f(w.z), x1.x, t0); t1 = fmaf(h2f(w.z >> 16), x1.y, t1);
          t0 = fmaf(h2f(w.w), x1.z, t0); t1 = fmaf(h2f(w.w >> 16), x1.w, t1);
          acc[k] += t0 + t1;
        }
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(xs.xf + c);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const u32x4 w = raw[k].v[i];
          float t0 = __uint_as_float(w.x) * x0.x, t1 = __uint_as_float(w.y) * x0.y;
          t0 = fmaf(__uint_as_float(w.z), x0.z, t0); t1 = fmaf(__uint_as_float(w.w), x0.w, t1);
          acc[k] += t0 + t1;
        }
      }
    }
  }
};
typedef FloatF<true> F16F;
typedef FloatF<false> F32F;

// ------------------------------------------------------------------ kernel

// Rows per work item and items in flight per wave on the register path: the gate/up pair
// carries two rows already; the q/k/v launch needs RoPE pairs (2 rows) in one item.
template <int EPI>
constexpr int GEMV_DEPTH = EPI == EPI_QKV ? NT_GEMV_DEPTH_QKV : EPI == EPI_SWIGLU ? NT_GEMV_DEPTH_PAIR : NT_GEMV_DEPTH;
template <int EPI>
constexpr int GEMV_ROWS = (EPI == EPI_SWIGLU) ? 1 : (EPI == EPI_QKV) ? 2 : NT_GEMV_ROWS;

// Power-of-two staging scale of a 32-column block whose largest |x| has the bit pattern mb
// (of a non-negative float, NaN included): the smallest s = 2^e with max |x| / s <= 127.
// Returns su = s / 256^(XL-1) (the stored scale) and k = 1 / su, which maps x to its
// fixed-point value X.  e is kept >= -100, so both stay normal numbers.  A block holding a
// NaN or an infinity gets scale NaN, so the rows it meets come out NaN.
__device__ __forceinline__ void limb_scale(uint32_t mb, float& su, float& k) {
  int E = (int)(mb >> 23) - 127;  // exponent of max |x| (-127 for 0 and subnormals)
  E = E < -100 ? -100 : E;
  int e = E - 6;                  // max |x| / 2^(E-6) lies in [64, 128)
  if (__uint_as_float(mb) * __uint_as_float((uint32_t)(127 - e) << 23) > 127.f) ++e;
  constexpr int FB = 8 * (XL - 1);
  su = mb >= 0x7F800000u ? __uint_as_float(0x7FC00000u) : __uint_as_float((uint32_t)(127 + e - FB) << 23);
  k = __uint_as_float((uint32_t)(127 + FB - e) << 23);
}

// bytes 0 of a, b, c, d -> one dword, a in the lowest byte
__device__ __forceinline__ uint32_t pack_b0(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0C0C0400u), hi = __builtin_amdgcn_perm(d, c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// The limb digits of four consecutive columns v[0..3] (k from limb_scale): dword i of each
// limb plane l of w.  The last limb is the low byte of X, the middle one (three limbs) the
// low byte of (X + 128) >> 8, the first (X + 128 (+ 32768)) >> 8 (XL - 1): each digit is
// the signed byte that leaves the rest divisible by 256.
template <int N>
__device__ __forceinline__ void limb_digits(const float* v, float k, uint32_t (&w)[XL][N], int i) {
  uint32_t b[XL][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int X = (int)rintf(v[j] * k);
    b[XL - 1][j] = (uint32_t)X;
    if constexpr (XL == 3) {
      b[1][j] = (uint32_t)((X + 128) >> 8);
      b[0][j] = (uint32_t)((X + 32896) >> 16);
    } else {
      b[0][j] = (uint32_t)((X + 128) >> 8);
    }
  }
#pragma unroll
  for (int l = 0; l < XL; ++l) w[l][i] = pack_b0(b[l][0], b[l][1], b[l][2], b[l][3]);
}

// x and gain of this thread's first 16 columns, loaded before a wave issues its first weight
// loads: loads complete in issue order, so staging from loads issued after the weights would
// wait for the weights.  Threads past the last group load the last group (unused).
struct XPre {
  float4 v[4], g[4];
};
__device__ __forceinline__ XPre stage_x_load(const GemvArgs& a) {
  XPre p;
  const int gi = min((int)threadIdx.x, (a.cols >> 4) - 1);
  const float4* src = reinterpret_cast<const float4*>(a.x + gi * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) p.v[i] = src[i];
  // loaded even without a gain (then from x, unused), so that the loads in flight do not
  // depend on the branch and the staging can wait for x alone
  const float4* gp = reinterpret_cast<const float4*>((a.gain ? a.gain : a.x) + gi * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) p.g[i] = gp[i];
  return p;
}

// One group of 16 columns (already normalised) into the limb planes, its sum and, from the
// even thread of each pair, the pair's scale.
__device__ __forceinline__ void stage_group(const XLimbs& xs, int gi, const float (&v)[16]) {
  if (xs.xf) {
    float4* d = reinterpret_cast<float4*>(xs.xf + gi * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  }
  float sum = 0.f;
  uint32_t mb = 0;  // max of |x| as bit patterns: a NaN orders above every number
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    sum += v[i] + v[i + 1];
    mb = max(mb, max(__float_as_uint(v[i]) & 0x7FFFFFFFu, __float_as_uint(v[i + 1]) & 0x7FFFFFFFu));
  }
  xs.s16[gi] = sum;
  mb = max(mb, (uint32_t)__builtin_amdgcn_mov_dpp((int)mb, 0xB1, 0xF, 0xF, true));  // the pair's 32 columns
  float s, k;
  limb_scale(mb, s, k);
  if ((gi & 1) == 0) xs.sc[gi >> 1] = s;
  if (!xs.q) return;
  uint32_t w[XL][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) limb_digits(&v[4 * i], k, w, i);
#pragma unroll
  for (int l = 0; l < XL; ++l)
    *reinterpret_cast<u32x4a16*>(xs.q + l * xs.plane + xq_off(gi * 16)) = u32x4a16{w[l][0], w[l][1], w[l][2], w[l][3]};
}

// Stage x into LDS: XL limb planes, the scale of every 32 columns and the fp32 sum of
// every 16.  Every thread of the workgroup calls this exactly once, with what stage_x_load
// returned.  A thread takes 16 columns per round, the first round from the preloaded
// registers; threads 2t and 2t+1 (one DPP quad pair) share a scale.  cols / 16 is even and
// the block size a multiple of 64, so both threads of a pair run the same rounds.
// With a gain the launch computes W (r x * g) for the RMSNorm factor r = 1 / sqrt(mean(x^2)
// + eps): x * g is staged as it arrives and r, a scalar per token, multiplies each row's dot
// product instead (W (r v) = r (W v); the limbs' power-of-two scale per 32 columns makes
// their precision independent of r), so the limbs do not wait for the workgroup's sum of
// squares.  Returns r (1 without a gain), valid after the staging's closing barrier.
__device__ __forceinline__ float stage_x(const GemvArgs& a, const XPre& pre, const XLimbs& xs, float* red) {
  const int cols = a.cols, ng = cols >> 4;
  const int g0 = (int)threadIdx.x;
  if (a.gain) {
    float ss = 0.f;
    if (g0 < ng) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ss += pre.v[i].x * pre.v[i].x + pre.v[i].y * pre.v[i].y + pre.v[i].z * pre.v[i].z + pre.v[i].w * pre.v[i].w;
    }
    for (int c = (g0 + (int)blockDim.x) * 16; c < cols; c += blockDim.x * 16) {
      const float4* src = reinterpret_cast<const float4*>(a.x + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 t = src[i];
        ss += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
      }
    }
    // this wave's part of the sum of squares; the waves' parts are added after the barrier
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  }
  if (g0 < ng) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 t = pre.v[i];
      if (a.gain) {
        t.x *= pre.g[i].x; t.y *= pre.g[i].y; t.z *= pre.g[i].z; t.w *= pre.g[i].w;
      }
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    stage_group(xs, g0, v);
  }
  for (int gi = g0 + (int)blockDim.x; gi < ng; gi += blockDim.x) {
    const float4* src = reinterpret_cast<const float4*>(a.x + gi * 16);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 t = src[i];
      if (a.gain) {
        const float4 g = reinterpret_cast<const float4*>(a.gain + gi * 16)[i];
        t.x *= g.x; t.y *= g.y; t.z *= g.z; t.w *= g.w;
      }
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    stage_group(xs, gi, v);
  }
  __syncthreads();
  if (!a.gain) return 1.f;
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return 1.0f / sqrtf(t / (float)cols + a.eps);
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

// Instruction-issue priority of this wave (0..3).  A SIMD's arbiter favours higher priority,
// then older waves, so with equal static shares the waves that start later fall behind and
// finish last; a wave that lowers its priority as its own remaining share shrinks lets the
// waves that are behind take the issue slots, and the waves of a CU end closer together.
__device__ __forceinline__ void set_wave_priority(int p) {
  if (p >= 3) __builtin_amdgcn_s_setprio(3);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// This wave's groups of R rows of one segment: group grp0 + k for k = wave_id, wave_id + W, ...
// over the launch's W waves.  The loads of the next step (or of the next group's first
// step) are in flight while the current step computes.  For the first segment the wave
// issues its first loads before the workgroup stages x, so that both latencies overlap;
// every wave takes part in the staging.
// DEPTH - 1 items in flight ahead of the one computed, in a ring of DEPTH register buffers
// (unrolled over the ring, so that no buffer is copied).
template <typename F, int R, int EPI, int DEPTH, bool STAGE>
__device__ __forceinline__ void run_segment(const GemvArgs& a, int s, int lane, int wid, int W, const XLimbs& xs,
                                            float* red, float& xscale, unsigned long long& best, const float2* rope,
                                            const XPre xpre) {
  constexpr int NR = (EPI == EPI_SWIGLU) ? 2 * R : R;
  typedef typename F::Raw Raw;
  const GemvSeg sg = a.seg[s];
  const int n_groups = (sg.rows + R - 1) / R;
  int k0 = (wid - sg.grp0) % W;
  if (k0 < 0) k0 += W;
  const int nsteps = F::steps(a.cols);
  // this wave's work items, in order: (group k0 + i W, step t) for i = 0, 1, ... and t = 0..nsteps-1
  const int n_items = (k0 < n_groups) ? ((n_groups - 1 - k0) / W + 1) * nsteps : 0;
  // a later segment without work for this wave is skipped whole (the first one stages x,
  // which every wave takes part in)
  if constexpr (!STAGE) {
    if (n_items == 0) return;
  }

  // load cursor: the item whose blocks are loaded next (DEPTH - 1 items ahead of the one computed)
  int lk = k0, lt = 0;
  auto issue = [&](Raw (&buf)[NR]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int r = min(lk * R + j, sg.rows - 1);  // past-the-end rows re-read the last row; results dropped
      buf[j] = F::load(sg.w + (size_t)r * sg.row_bytes, a.cols, lt, lane);
      if constexpr (EPI == EPI_SWIGLU) buf[R + j] = F::load(a.seg[1].w + (size_t)r * sg.row_bytes, a.cols, lt, lane);
    }
    if (++lt == nsteps) {
      lt = 0;
      lk += W;
    }
  };
  Raw b0[NR], b1[NR], b2[NR];
  // issued even by a wave without items (clamped rows; segments have at least one row), so
  // that the count in flight is static and the staging's waits leave these loads in flight
  issue(b0);
  if (DEPTH == 3) issue(b1);
  if constexpr (STAGE) xscale = stage_x(a, xpre, xs, red);
  if (n_items == 0) return;
  float acc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) acc[j] = 0.f;
  int ck = k0, ct = 0, item = 0;  // compute cursor
  // compute the item in `cur` while the DEPTH - 1 after it are in flight; refill the buffer
  // that the previous item used
  auto step = [&](const Raw (&cur)[NR], Raw (&refill)[NR]) -> bool {
    // unconditional (past the last item the loads re-read clamped rows), so that the count
    // of loads in flight is static and the wait for this item leaves the later ones in flight
    issue(refill);
    F::template fma<NR>(cur, a.cols, ct, lane, xs, acc);
    if (ct == nsteps - 1) {
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = wave_sum(acc[j]) * xscale;
      epilogue<R, EPI>(a, s, sg, ck * R, lane, acc, best, rope);
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = 0.f;
    }
    if (++ct == nsteps) {
      ct = 0;
      ck += W;
    }
    // priority from the remaining fraction of this segment's items: 3 for the first quarter,
    // then 2, 1, 0
    ++item;
    set_wave_priority((4 * (n_items - item)) / (n_items + 1));
    return item < n_items;
  };
  set_wave_priority(3);
  if constexpr (DEPTH == 3) {
    for (;;) {
      if (!step(b0, b2)) break;
      if (!step(b1, b0)) break;
      if (!step(b2, b1)) break;
    }
  } else {
    for (;;) {
      if (!step(b0, b1)) break;
      if (!step(b1, b0)) break;
    }
  }
}

// Format "masks" of the kernels instantiated for q/k/v launches whose segments are Q4_K,
// Q4_K, Q6_K or Q5_K, Q5_K, Q6_K or Q4_KT, Q4_KT, Q6_K in that order (the Q4_K_M and Q5_K_M
// layers).
constexpr int FMTS_Q4K_Q4K_Q6K = 1 << 12;
constexpr int FMTS_Q5K_Q5K_Q6K = 1 << 13;
constexpr int FMTS_Q4KT_Q4KT_Q6K = 1 << 14;
// With a Q4_KT or Q8_0T segment: its loads take the nontemporal policy (launches of at least
// 10^8 weights).
constexpr int FMT_NTL = 1 << 15;
constexpr bool is_fixed_qkv(int m) { return m == FMTS_Q4K_Q4K_Q6K || m == FMTS_Q5K_Q5K_Q6K || m == FMTS_Q4KT_Q4KT_Q6K; }

// Segment s with its format's work loop (STAGE: the first segment, which stages x).
template <int FMTMASK, int R, int EPI, bool STAGE>
__device__ __forceinline__ void run_any(const GemvArgs& a, int s, int lane, int wid, int W, const XLimbs& xs,
                                        float* red, float& xscale, unsigned long long& best, const float2* rope, const XPre xpre) {
  constexpr int D = GEMV_DEPTH<EPI>;
  switch (a.seg[s].fmt) {
    case FMT_Q8_0:
      if constexpr ((FMTMASK >> FMT_Q8_0) & 1) run_segment<Q8_0F, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q4_0:
      if constexpr ((FMTMASK >> FMT_Q4_0) & 1) run_segment<Q4_0F, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q4_K:
      if constexpr ((FMTMASK >> FMT_Q4_K) & 1) run_segment<Q4_KF, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q5_KT:
      if constexpr ((FMTMASK >> FMT_Q5_KT) & 1)
        run_segment<Q5_KTF<(FMTMASK & FMT_NTL) != 0>, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q8_0T:
      if constexpr ((FMTMASK >> FMT_Q8_0T) & 1)
        run_segment<Q8_0TF<(FMTMASK & FMT_NTL) != 0>, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q4_KT:
      if constexpr ((FMTMASK >> FMT_Q4_KT) & 1)
        run_segment<Q4_KTF<(FMTMASK & FMT_NTL) != 0>, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_Q5_K:
      if constexpr ((FMTMASK >> FMT_Q5_K) & 1) run_segment<Q5_KF, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_F16:
      if constexpr ((FMTMASK >> FMT_F16) & 1) run_segment<F16F, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    case FMT_F32:
      if constexpr ((FMTMASK >> FMT_F32) & 1) run_segment<F32F, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
    default:
      if constexpr ((FMTMASK >> FMT_Q6_K) & 1) run_segment<Q6_KF, R, EPI, D, STAGE>(a, s, lane, wid, W, xs, red, xscale, best, rope, xpre);
      break;
  }
}

// At least four waves per SIMD (at most 128 VGPRs): the stream needs many waves in flight.
// Which staged forms of x a launch's formats read: the limbs (quantized formats) and/or the
// fp32 copy (F16, F32).
constexpr bool mask_has_q(int m) { return (m & (0x1F | (1 << FMT_Q4_KT) | (1 << FMT_Q8_0T) | (1 << FMT_Q5_KT) | FMTS_Q4K_Q4K_Q6K | FMTS_Q5K_Q5K_Q6K | FMTS_Q4KT_Q4KT_Q6K)) != 0; }
constexpr bool mask_has_f(int m) { return (m & ((1 << FMT_F16) | (1 << FMT_F32))) != 0; }

template <int FMTMASK, int R, int NW, int EPI>
__global__ __launch_bounds__(NW * 64, 4) void gemv_kernel(const GemvArgs a) {
  extern __shared__ float4 smem4[];
  XLimbs xs;
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem4);
  xs.plane = xq_plane(a.cols);
  xs.q = mask_has_q(FMTMASK) ? lds : nullptr;
  lds += mask_has_q(FMTMASK) ? XL * xs.plane : 0;
  xs.xf = mask_has_f(FMTMASK) ? reinterpret_cast<float*>(lds) : nullptr;
  lds += mask_has_f(FMTMASK) ? 4 * a.cols : 0;
  xs.sc = reinterpret_cast<float*>(lds);
  xs.s16 = xs.sc + (a.cols >> 5);
  float* red = xs.s16 + (a.cols >> 4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wid = (int)blockIdx.x * NW + wave;
  const int W = (int)gridDim.x * NW;
  unsigned long long best = 0;
  float xscale = 1.f;  // the RMSNorm factor, set by the staging of x (first segment)
  // RoPE table for this position (visible after the barrier inside the staging of x)
  __shared__ float2 rope[64];
  if constexpr (EPI == EPI_QKV) {
    if (threadIdx.x < 64) rope[threadIdx.x] = rope_cs(a.rope_theta, a.pos, threadIdx.x, 128);
  }
  // x is loaded first (its loads then complete before the weights'); the first segment
  // stages it after issuing its first weight loads
  const XPre xpre = stage_x_load(a);
  if constexpr (is_fixed_qkv(FMTMASK)) {
    // the three segments' formats fixed at compile time: straight-line code, so registers
    // are allocated per segment rather than for every format at every segment
    constexpr int D = GEMV_DEPTH<EPI>;
    using FK = std::conditional_t<FMTMASK == FMTS_Q4K_Q4K_Q6K, Q4_KF,
                                  std::conditional_t<FMTMASK == FMTS_Q4KT_Q4KT_Q6K, Q4_KTF<false>, Q5_KF>>;
    run_segment<FK, R, EPI, D, true>(a, 0, lane, wid, W, xs, red, xscale, best, rope, xpre);
    run_segment<FK, R, EPI, D, false>(a, 1, lane, wid, W, xs, red, xscale, best, rope, XPre{});
    run_segment<Q6_KF, R, EPI, D, false>(a, 2, lane, wid, W, xs, red, xscale, best, rope, XPre{});
  } else {
    run_any<FMTMASK, R, EPI, true>(a, 0, lane, wid, W, xs, red, xscale, best, rope, xpre);
    const int nseg = (EPI == EPI_SWIGLU) ? 1 : a.nseg;
    for (int s = 1; s < nseg; ++s) run_any<FMTMASK, R, EPI, false>(a, s, lane, wid, W, xs, red, xscale, best, rope, XPre{});
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


// ================================================================== k-token GEMM
//
// Y[t] = W X[t] for t < n_tok tokens at once (the verification pass of self-speculative
// decoding: the draft tokens, which come from the VRAM-resident layers, meet every weight
// of the full model in one pass; ntransformer overview, de.news.hada.io,
// "Hauptfunktionen").  The register path with a token dimension: a workgroup stages the
// NT activation vectors as limbs, one LDS region each; a wave's row blocks are loaded once
// per step and dotted with every token's limbs (the code unpacking is shared: it depends
// on the loaded bytes only), so the weights are read once for all NT tokens.  Tokens past
// n_tok are staged as zeros and never stored.  A launch covers a column chunk: the host
// splits wide matrices so that NT chunks of x fit in LDS, and every chunk after the first
// adds into Y (stream order separates the chunks).

struct GemmArgs {
  const uint8_t* w;  // first block of the chunk in row 0
  int64_t row_bytes; // of the whole matrix
  int rows;
  int cols;          // of the chunk
  int n_tok;
  const float* x;    // token 0's chunk; token t at x + t * xld
  int64_t xld;
  float* y;          // token t's outputs at y + t * yld
  int64_t yld;
  int accum;         // add into y
};

// Q4_K and Q5_K in the k-token GEMM: an item's codes (four 8-bit codes per dword, per run
// of 16 columns) and its scale factors d sc and dmin m are decoded once and then dotted
// with each token's limbs, so that the unpacking is not repeated per token.
template <int NR>
struct KDec {
  uint32_t code[NR][4][4];  // [row][run h][dword]
  float dA[NR], dB[NR], mA[NR], mB[NR];  // d sc and dmin m of sub-blocks 2g and 2g + 1
  int c0;
  bool ok;
};

template <typename F, int NR>
__device__ __forceinline__ void kdecode(const typename F::Raw (&raw)[NR], int cols, int step, int lane, KDec<NR>& D) {
  constexpr bool K5 = std::is_base_of<Q5_KF, F>::value;
  const int sb = step * 16 + (lane >> 2);
  D.ok = sb < (cols >> 8);
  const int g = lane & 3;
  D.c0 = (sb << 8) + (g << 6);
  const uint32_t m0f = 0x0F0F0F0Fu, m10 = 0x10101010u;
  const uint32_t rot_a = (uint32_t)(2 * g + 28) & 31u, rot_b = (uint32_t)(2 * g + 29) & 31u;
#pragma unroll
  for (int k = 0; k < NR; ++k)
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t v = (h & 1) ? raw[k].qb[i] : raw[k].qa[i];
        uint32_t c = h < 2 ? (v & m0f) : ((v >> 4) & m0f);
        if constexpr (K5) {
          const uint32_t hv = (h & 1) ? raw[k].hb[i] : raw[k].ha[i];
          c = and_or(__builtin_amdgcn_alignbit(hv, hv, h < 2 ? rot_a : rot_b), m10, c);
        }
        D.code[k][h][i] = c;
      }
  // the 6-bit scales and mins of sub-blocks 2g, 2g + 1, gathered as in the GEMV formats
  const uint32_t p = 2u * (uint32_t)(g & 1);
  const uint32_t sel = p | ((p + 1) << 8) | ((p + 4) << 16) | ((p + 5) << 24);
  const bool upper = g >= 2;
  const uint32_t mlow = upper ? 0x0F0F0F0Fu : 0x3F3F3F3Fu, mtop = upper ? 0x30303030u : 0u;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const uint32_t Y = raw[k].hd.y, Z = raw[k].hd.z, W = raw[k].hd.w;
    const uint32_t yz = __builtin_amdgcn_perm(Z, Y, sel);
    const uint32_t lo = upper ? __builtin_amdgcn_perm(W >> 4, W, sel) : yz;
    const uint32_t sm = and_or(yz >> 2, mtop, lo & mlow);
    const float d = h2f(raw[k].hd.x), dmin = h2f(raw[k].hd.x >> 16);
    D.dA[k] = d * ub0(sm);
    D.dB[k] = d * ub1(sm);
    D.mA[k] = dmin * ub2(sm);
    D.mB[k] = dmin * ub3(sm);
  }
}

template <int NR>
__device__ __forceinline__ void kapply(const KDec<NR>& D, const XLimbs& xs, float (&acc)[NR]) {
  if (!D.ok) return;
  int da[NR][XL], db[NR][XL];
  zero_limbs(da);
  zero_limbs(db);
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const XRun x = x_run(xs, D.c0 + 16 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < NR; ++k) dot_limbs(D.code[k][h][i], x, i, h < 2 ? da[k] : db[k], (h & 1) == 0 && i == 0);
  }
  const float sA = xs.sc[D.c0 >> 5], sB = xs.sc[(D.c0 >> 5) + 1];
  const float4 x4 = s16x4(xs, D.c0);
  const float xa = x4.x + x4.y, xb = x4.z + x4.w;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    acc[k] += (D.dA[k] * sA) * limb_sum(da[k]);
    acc[k] += (D.dB[k] * sB) * limb_sum(db[k]);
    acc[k] -= D.mA[k] * xa + D.mB[k] * xb;
  }
}

template <typename F, int NT, int R>
__device__ __forceinline__ void gemm_rows(const GemmArgs& a, const XLimbs (&xs)[NT], int lane, int wid, int W) {
  typedef typename F::Raw Raw;
  const int n_groups = (a.rows + R - 1) / R;
  const int nsteps = F::steps(a.cols);
  const int n_items = wid < n_groups ? ((n_groups - 1 - wid) / W + 1) * nsteps : 0;
  if (n_items == 0) return;
  int lk = wid, lt = 0;
  auto issue = [&](Raw (&buf)[R]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int r = min(lk * R + j, a.rows - 1);  // past-the-end rows re-read the last row; results dropped
      buf[j] = F::load(a.w + (size_t)r * a.row_bytes, a.cols, lt, lane);
    }
    if (++lt == nsteps) {
      lt = 0;
      lk += W;
    }
  };
  Raw b0[R], b1[R];
  issue(b0);
  float acc[NT][R];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[t][j] = 0.f;
  int ck = wid, ct = 0, item = 0;
  auto step = [&](const Raw (&cur)[R], Raw (&refill)[R]) -> bool {
    issue(refill);  // unconditional: the wait for this item leaves the next one in flight
    if constexpr (std::is_base_of<Q4_KF, F>::value || std::is_base_of<Q5_KF, F>::value) {
      KDec<R> dec;
      kdecode<F, R>(cur, a.cols, ct, lane, dec);
#pragma unroll
      for (int t = 0; t < NT; ++t) kapply<R>(dec, xs[t], acc[t]);
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) F::template fma<R>(cur, a.cols, ct, lane, xs[t], acc[t]);
    }
    if (ct == nsteps - 1) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int j = 0; j < R; ++j) acc[t][j] = wave_sum(acc[t][j]);
        const int r = ck * R + lane;
        if (t < a.n_tok && lane < R && r < a.rows) {
          float v = acc[t][0];
#pragma unroll
          for (int j = 1; j < R; ++j) v = (lane == j) ? acc[t][j] : v;
          float* yp = a.y + (size_t)t * a.yld + r;
          *yp = a.accum ? *yp + v : v;
        }
#pragma unroll
        for (int j = 0; j < R; ++j) acc[t][j] = 0.f;
      }
    }
    if (++ct == nsteps) {
      ct = 0;
      ck += W;
    }
    return ++item < n_items;
  };
  for (;;) {
    if (!step(b0, b1)) break;
    if (!step(b1, b0)) break;
  }
}

// Stage token t's chunk of x (zeros for t >= n_tok) into its limb region: a thread takes
// 16 columns per round, as stage_x does, without a norm.
__device__ __forceinline__ void gemm_stage(const GemmArgs& a, int t, const XLimbs& xs, int nthreads) {
  const int ng = a.cols >> 4;
  const float* x = a.x + (size_t)t * a.xld;
  for (int gi = (int)threadIdx.x; gi < ng; gi += nthreads) {
    float v[16];
    if (t < a.n_tok) {
      const float4* src = reinterpret_cast<const float4*>(x + gi * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 q = src[i];
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.f;
    }
    stage_group(xs, gi, v);
  }
}

// Rows per item: two, or one where two rows' loads in both ring buffers, the decoded codes
// and NT tokens' accumulators would not fit the registers (Q5_K: five 128-bit loads per row;
// Q4_K from two tokens on; Q6_K at 8 tokens).
template <int FMT, int NT>
constexpr int GEMM_ROWS = (FMT == FMT_Q5_K || FMT == FMT_Q5_KT || ((FMT == FMT_Q4_K || FMT == FMT_Q4_KT) && NT >= 2) || (FMT == FMT_Q6_K && NT == 8)) ? 1 : 2;

template <int FMT, int NT, int NW>
__global__ __launch_bounds__(NW * 64, 4) void gemm_kernel(const GemmArgs a) {
  extern __shared__ float4 smem4[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wid = (int)blockIdx.x * NW + wave;
  const int W = (int)gridDim.x * NW;
  constexpr bool FF = is_float_fmt(FMT);
  const size_t per_tok = gemm_lds_per_token(a.cols, FF);
  XLimbs xs[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint8_t* base = reinterpret_cast<uint8_t*>(smem4) + t * per_tok;
    xs[t].plane = xq_plane(a.cols);
    xs[t].q = FF ? nullptr : base;
    xs[t].xf = FF ? reinterpret_cast<float*>(base) : nullptr;
    xs[t].sc = reinterpret_cast<float*>(base + (FF ? sizeof(float) * a.cols : (size_t)XL * xs[t].plane));
    xs[t].s16 = xs[t].sc + (a.cols >> 5);
    gemm_stage(a, t, xs[t], NW * 64);
  }
  __syncthreads();
  constexpr int R = GEMM_ROWS<FMT, NT>;
  if constexpr (FMT == FMT_Q8_0) gemm_rows<Q8_0F, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q4_0) gemm_rows<Q4_0F, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q4_K) gemm_rows<Q4_KF, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q4_KT) gemm_rows<Q4_KTF<false>, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q8_0T) gemm_rows<Q8_0TF<false>, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q5_KT) gemm_rows<Q5_KTF<false>, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_Q5_K) gemm_rows<Q5_KF, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_F16) gemm_rows<F16F, NT, R>(a, xs, lane, wid, W);
  else if constexpr (FMT == FMT_F32) gemm_rows<F32F, NT, R>(a, xs, lane, wid, W);
  else gemm_rows<Q6_KF, NT, R>(a, xs, lane, wid, W);
}

// ---- k-token GEMM on the matrix cores (Q4_K, Q5_K and Q6_K, 3 to 8 tokens)
//
// The GEMV's limb arithmetic on v_mfma_i32_16x16x32_i8.  For one 32-column sub-block of a
// Q4_K superblock the A operand holds 16 rows of staged activation digits, row 4u + l being
// limb l of token 4m + u (row 4u + 3 is unused), and the B operand the 4-bit codes (as
// bytes) of 16 weight rows, so one instruction forms the exact integer sums
// D[(token, limb)][row] = sum over the 32 columns of digit * code for 16 weight rows and
// four tokens (|D| <= 32 * 128 * 15: exact in int32 and in fp32).  An A fragment is read
// from LDS once per wave and sub-block and serves 16 weight rows, where the VALU kernel
// reads every token's digits again for every row (its LDS-read bound).  A lane's four D
// values are the limbs of one token for its own weight row, so they combine in the lane
// exactly as the GEMV's limb_sum does, the row's d sc and dmin m are decoded once per lane,
// and each sub-block costs the lane one scaled FMA per token plus the min term (dmin m
// times the block's fp32 x sum, as in the GEMV).
//
// Operand layouts (8 bytes per lane): A lane l holds row l % 16 at k = 8 (l / 16) .. +7, B
// lane l column l % 16 at the same k, and D lane l rows 4 (l / 16) .. +3 of column l % 16.
// A and B only need the same assignment of the sub-block's 32 columns to (lane group q,
// byte): q takes bytes 8q .. 8q + 7 of the sub-block pair's 32 code bytes (low nibbles are
// sub-block 2g, high nibbles 2g + 1) and the digits of the same 8 columns.
//
// Work: one workgroup of 16 waves per CU walks 16-row tiles; the waves split a tile's
// superblocks (wave w takes superblocks w and w + 16 of a column chunk of at most 32) and
// write their per-(row, token) sums to LDS (two buffers, so one barrier per tile); 16 NT
// threads then add the 16 waves' sums and store the tile.  The next tile's loads are issued
// before the current tile is computed; one loop iteration is one tile, with the barrier in
// one place, so that the registers of the two tiles stay fixed (an unrolled ring of steps
// with the barrier in each step was merged back into one step by the compiler, which then
// waited for every load in flight at the top of the loop).

template <int FMT>
struct MmRaw;
template <>
struct MmRaw<FMT_Q4_K> {
  u32x2 q[4];  // code bytes 16 + 32 g + 8 q_lane .. +7 of the lane's row, g = 0..3
  u32x4 hd;    // d, dmin and the 12 packed scale/min bytes
};
// Q5_K: Q4_K's fields with the nibbles at 48 + 32 g and the fifth code bit of column l of
// sub-block j in bit j of high-bit byte 16 + l (the lane's columns 8 q_lane .. +7 of every
// sub-block share its eight high-bit bytes)
template <>
struct MmRaw<FMT_Q5_K> {
  u32x2 q[4];
  u32x2 qh;
  u32x4 hd;
};
// Q6_K: the lane's eight columns 8 q_lane .. +7 of each 32-column pair p of sub-blocks take
// low-bit bytes 64 h + 32 e + 8 q_lane .. +7 (h = p / 4, e = p % 2; nibble p / 2 % 2) and
// high-bit bytes 128 + 32 h + 8 q_lane .. +7 (bits 2 (p % 4) ..); superblocks sit at 2-byte
// phases (210 = 2 mod 4) and are read with loads at 2-byte alignment, which the runtime's
// unaligned access mode serves (a whole 16-byte piece where one straddles a line)
typedef uint32_t u32x2a2 __attribute__((ext_vector_type(2), aligned(2)));
typedef uint32_t u32x4a2 __attribute__((ext_vector_type(4), aligned(2)));
template <>
struct MmRaw<FMT_Q6_K> {
  u32x2 ql[4];  // [2 h + e]
  u32x2 qh[2];  // [h]
  u32x4 sc;     // the 16 int8 sub-block scales
  uint32_t d;   // fp16 d in the low half
};

#ifndef NT_MM_WAVES
#define NT_MM_WAVES 16
#endif
constexpr int MM_NW = NT_MM_WAVES;  // waves per workgroup of the matrix-core GEMM
constexpr int MM_SMAX = 32 / MM_NW;  // superblocks per wave and tile at the widest chunk (32)

// LDS: the tokens' limb regions, the digit scales per (32-column block, token), the x sums
// per (32-column block, token) for Q4_K's mins or per (16-column block, token) for Q6_K's
// offset, and two buffers of per-(wave, row, token) sums
__host__ __device__ __forceinline__ size_t mm_lds_bytes(int fmt, int nt, int cols) {
  const size_t xs = (size_t)nt * gemm_lds_per_token(cols);
  const size_t tr = (size_t)(fmt == FMT_Q6_K ? 3 : 2) * sizeof(float) * (size_t)(cols >> 5) * (size_t)nt;
  const size_t red = (size_t)2 * MM_NW * 16 * (size_t)nt * sizeof(float);
  return xs + ((tr + 15) & ~(size_t)15) + red;
}

template <int FMT, int NT, int S>
__global__ __launch_bounds__(MM_NW * 64, 1) void gemm_mfma_kernel(const GemmArgs a) {
  static_assert(FMT == FMT_Q4_K || FMT == FMT_Q5_K || FMT == FMT_Q6_K, "Q4_K, Q5_K or Q6_K");
  constexpr bool K6 = FMT == FMT_Q6_K, K5 = FMT == FMT_Q5_K;
  static_assert(NT == 4 || NT == 8, "four tokens per MFMA");
  static_assert(S >= 1 && S <= 4, "superblocks per wave and tile");
  constexpr int NW = MM_NW, NM = NT / 4;
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ float4 smem4[];
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem4);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int iw = lane & 15, q = lane >> 4;
  const size_t per_tok = gemm_lds_per_token(a.cols);
  const int plane = xq_plane(a.cols);
  const int nblk = a.cols >> 5;
  // ---- stage every token's chunk of x as limbs (16 columns of one token per thread and
  // round, at most four rounds: NT * cols <= 2^16; every round's loads issued first), then
  // the digit scales and x sums per (32-column block, token), token-minor
  {
    const int ng = a.cols >> 4, total = NT * ng;  // ng even: a DPP pair stays in one token
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = (int)threadIdx.x + NW * 64 * u, t = i / ng, gi = i % ng;
      if (i < total && t < a.n_tok) {
        const float4* src = reinterpret_cast<const float4*>(a.x + (size_t)t * a.xld + gi * 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float4 f = src[k];
          v[u][4 * k] = f.x; v[u][4 * k + 1] = f.y; v[u][4 * k + 2] = f.z; v[u][4 * k + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) v[u][k] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = (int)threadIdx.x + NW * 64 * u, t = i / ng, gi = i % ng;
      if (i < total) {
        XLimbs xs;
        xs.q = lds + t * per_tok;
        xs.plane = plane;
        xs.sc = reinterpret_cast<float*>(xs.q + XL * plane);
        xs.s16 = xs.sc + nblk;
        stage_group(xs, gi, v[u]);
      }
    }
  }
  __syncthreads();
  float* scT = reinterpret_cast<float*>(lds + NT * per_tok);
  float* xsT = scT + nblk * NT;  // per 32 columns (Q4_K) or per 16 (Q6_K)
  float* red = reinterpret_cast<float*>(
      lds + NT * per_tok + (((size_t)(K6 ? 3 : 2) * sizeof(float) * nblk * NT + 15) & ~(size_t)15));
  for (int i = threadIdx.x; i < nblk * NT; i += NW * 64) {
    const int b = i / NT, t = i % NT;
    const float* sc = reinterpret_cast<const float*>(lds + t * per_tok + XL * plane);
    scT[i] = sc[b];
    if constexpr (K6) {
      xsT[2 * b * NT + t] = sc[nblk + 2 * b];
      xsT[(2 * b + 1) * NT + t] = sc[nblk + 2 * b + 1];
    } else {
      xsT[i] = sc[nblk + 2 * b] + sc[nblk + 2 * b + 1];
    }
  }
  __syncthreads();

  // ---- this lane's A rows: token 4m + iw / 4, limb iw % 4 (the unused fourth reads limb
  // XL - 1: real digits, whose sums are dropped); its outputs: token 4m + q
  const uint8_t* abase[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
    abase[m] = lds + (4 * m + (iw >> 2)) * per_tok + min(iw & 3, XL - 1) * plane + 8 * q;

  const int nsb = a.cols >> 8;  // at most NW * S
  const int ntiles = (a.rows + 15) >> 4;
  if ((int)blockIdx.x >= ntiles) return;
  const uint32_t m0f = 0x0F0F0F0Fu;
  // this wave's S superblocks of tile t (past the chunk's last superblock or the last row:
  // valid addresses whose results are dropped)
  auto issue = [&](MmRaw<FMT> (&r)[S], int t) {
    const int row = min(t * 16 + iw, a.rows - 1);
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int sb = min(wave + NW * k, nsb - 1);
      const uint8_t* p = a.w + (size_t)row * a.row_bytes + (size_t)sb * (K6 ? 210 : K5 ? 176 : 144);
      if constexpr (K6) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[k].ql[i] = *NT_GPTR(u32x2a2, p + 64 * (i >> 1) + 32 * (i & 1) + 8 * q);
#pragma unroll
        for (int h = 0; h < 2; ++h) r[k].qh[h] = *NT_GPTR(u32x2a2, p + 128 + 32 * h + 8 * q);
        r[k].sc = *NT_GPTR(u32x4a2, p + 192);
        r[k].d = wld2(p + 208);
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) r[k].q[g] = wld8(p + (K5 ? 48 : 16) + 32 * g + 8 * q);
        if constexpr (K5) r[k].qh = wld8(p + 16 + 8 * q);
        r[k].hd = wld16(p);
      }
    }
  };
  // lanes of lane groups 0-1 carry the first sub-block of a Q6_K pair, 2-3 the second
  const uint64_t half_a = q < 2 ? ~0ull : 0ull, half_b = ~half_a;
  (void)half_a;
  (void)half_b;
  int ct = blockIdx.x, buf = 0;
  // one tile: the next tile's loads go into the other buffer and stay in flight while this
  // one is computed (the two buffers alternate, so no register copy waits for them)
  auto tile = [&](const MmRaw<FMT> (&cur)[S], MmRaw<FMT> (&nxt)[S]) -> bool {
    const int tn = ct + (int)gridDim.x;
    issue(nxt, min(tn, ntiles - 1));
    float acc[NM], am[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = am[m] = 0.f;
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int sb = wave + NW * k;
      if (sb >= nsb) continue;
      if constexpr (K6) {
        const MmRaw<FMT_Q6_K>& c = cur[k];
        const float d = h2f(c.d);
        const uint32_t m30 = 0x30303030u;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {  // pair of sub-blocks 2 pp, 2 pp + 1: columns 32 pp ..
          const int h = pp >> 2, kk = pp & 3;
          const u32x2 lv = c.ql[2 * h + (kk & 1)], hv = c.qh[h];
          const uint32_t sl = 4u * (uint32_t)(kk >> 1), rot = (uint32_t)(2 * kk + 28) & 31u;
          const uint32_t c0 = and_or(__builtin_amdgcn_alignbit(hv.x, hv.x, rot), m30, (lv.x >> sl) & m0f);
          const uint32_t c1 = and_or(__builtin_amdgcn_alignbit(hv.y, hv.y, rot), m30, (lv.y >> sl) & m0f);
          const uint64_t code = ((uint64_t)c1 << 32) | c0;
          const long BA = (long)(code & half_a), BB = (long)(code & half_b);
          const uint32_t sw = pp < 2 ? c.sc.x : pp < 4 ? c.sc.y : pp < 6 ? c.sc.z : c.sc.w;
          const int sh = 16 * (pp & 1);
          const float dsa = d * (float)(int)(int8_t)(sw >> sh), dsb = d * (float)(int)(int8_t)(sw >> (sh + 8));
          const int cc = 256 * sb + 32 * pp;
          const int xo = xq_off(cc);
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const long A = *reinterpret_cast<const long*>(abase[m] + xo);
            const i32x4 DA = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, BA, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const i32x4 DB = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, BB, i32x4{0, 0, 0, 0}, 0, 0, 0);
            const int ti = (cc >> 5) * NT + 4 * m + q, t16 = (cc >> 4) * NT + 4 * m + q;
            const int la[XL] = {DA[0], DA[1], DA[XL - 1]}, lb[XL] = {DB[0], DB[1], DB[XL - 1]};
            const float sx = scT[ti];
            acc[m] = fmaf(dsa * sx, limb_sum(la), acc[m]);
            acc[m] = fmaf(dsb * sx, limb_sum(lb), acc[m]);
            am[m] = fmaf(dsa, xsT[t16], am[m]);  // w = d s (q - 32): the offset times the x sums
            am[m] = fmaf(dsb, xsT[t16 + NT], am[m]);
          }
        }
      } else {
      const MmRaw<FMT>& c = cur[k];
      const float d = h2f(c.hd.x), dmin = h2f(c.hd.x >> 16);
      const uint32_t Y = c.hd.y, Z = c.hd.z, W = c.hd.w;
      const uint32_t scA = Y & 0x3F3F3F3Fu, mA = Z & 0x3F3F3F3Fu;
      const uint32_t scB = (W & m0f) | ((Y >> 2) & 0x30303030u);
      const uint32_t mB = ((W >> 4) & m0f) | ((Z >> 2) & 0x30303030u);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sw = j < 4 ? scA : scB, mw = j < 4 ? mA : mB;
        const int sh = 8 * (j & 3);
        const float dsc = d * (float)((sw >> sh) & 0xFFu), dm = dmin * (float)((mw >> sh) & 0xFFu);
        const u32x2 v = c.q[j >> 1];
        uint32_t c0 = (j & 1) ? ((v.x >> 4) & m0f) : (v.x & m0f);
        uint32_t c1 = (j & 1) ? ((v.y >> 4) & m0f) : (v.y & m0f);
        if constexpr (K5) {  // bit j of each high-bit byte rotated into bit 4: codes 0..31
          const uint32_t m10 = 0x10101010u, rj = (uint32_t)(j + 28) & 31u;
          c0 = and_or(__builtin_amdgcn_alignbit(c.qh.x, c.qh.x, rj), m10, c0);
          c1 = and_or(__builtin_amdgcn_alignbit(c.qh.y, c.qh.y, rj), m10, c1);
        }
        const long B = (long)(((uint64_t)c1 << 32) | c0);
        const int cc = 256 * sb + 32 * j;  // first column of the sub-block in the chunk
        const int xo = xq_off(cc);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const long A = *reinterpret_cast<const long*>(abase[m] + xo);
          const i32x4 D = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
          const int ti = (cc >> 5) * NT + 4 * m + q;
          const int dl[XL] = {D[0], D[1], D[XL - 1]};
          acc[m] = fmaf(dsc * scT[ti], limb_sum(dl), acc[m]);
          am[m] = fmaf(dm, xsT[ti], am[m]);
        }
      }
      }
    }
    // ---- every lane holds its row's sums for tokens 4m + q; the waves meet in LDS
    float* rb = red + (size_t)buf * (NW * 16 * NT);
#pragma unroll
    for (int m = 0; m < NM; ++m) rb[(wave * 16 + iw) * NT + 4 * m + q] = acc[m] - (K6 ? 32.f : 1.f) * am[m];
    __syncthreads();
    if ((int)threadIdx.x < 16 * NT) {
      const int rr = threadIdx.x / NT, t = threadIdx.x % NT;
      const int row = ct * 16 + rr;
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) y += rb[(w * 16 + rr) * NT + t];
      if (row < a.rows && t < a.n_tok) {
        float* yp = a.y + (size_t)t * a.yld + row;
        *yp = a.accum ? *yp + y : y;
      }
    }
    buf ^= 1;  // the other buffer: the next tile's writes cannot meet this tile's reads
    ct = tn;
    return ct < ntiles;
  };
  MmRaw<FMT> b0[S], b1[S];
  issue(b0, ct);
  for (;;) {
    if (!tile(b0, b1)) break;
    if (!tile(b1, b0)) break;
  }
}

// ================================================================== streamed GEMV
//
// Column-stationary layout for shapes whose rows are 16-byte aligned.  A workgroup owns a
// contiguous range of row tasks; its waves split the columns into slices (4096 columns
// for the 256-weight superblock formats, 2048 for the 32-weight block formats) and, when
// a slice leaves waves over, split the tasks among them.  Each wave
//  * holds its slice of x in registers (64 or 32 floats per lane, loaded once), so x is
//    neither staged in LDS nor re-read per weight;
//  * streams the slice bytes of its rows from HBM into its own LDS ring with 16-byte
//    global->LDS transfers (global_load_lds_dwordx4): every transfer instruction reads
//    1 KiB of consecutive bytes, and D rows are in flight without costing registers;
//  * reads each row's pieces from LDS in the lane layout its format wants (unaligned
//    fields realigned with v_alignbyte), forms the lane's partial dot product and
//    reduces it over the wave; the slices of a row meet in LDS at the end.
// Lane layouts: superblock formats, lane = quarter g of superblock s (s = lane / 4):
// columns 256 s + 64 g .. + 63 of the slice; block formats, lane = block: 32 columns.

constexpr int ST_SLICE_COLS_K = 4096;
constexpr int ST_SLICE_COLS_B = 2048;
constexpr int ST_MAX_WAVES = 16;

// The streamed path's global->LDS transfers read 1 KiB of consecutive bytes per instruction,
// each line once, and take the nontemporal policy (cache-policy bits 2 = nt): the Q6_K down
// GEMV 42.6 vs 44.9 us, an 8B Q8_0 layer 3% faster.  (The register path's weight loads touch
// a line from two instructions and were 20-45% slower with it.)
#ifndef NT_STREAM_CPOL
#define NT_STREAM_CPOL 2
#endif
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, NT_STREAM_CPOL);
}
// the same with a cached read (data that other workgroups read too)
__device__ __forceinline__ void dma16c(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
__device__ __forceinline__ uint32_t lds4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ u32x4 lds16a(const uint8_t* p) {
  const u32x4a16 v = *reinterpret_cast<const u32x4a16*>(p);
  return u32x4{v.x, v.y, v.z, v.w};
}
// o[k] = the 4 bytes at p + 4k, where p sits `phase` (0 or 2) bytes past a 4-byte boundary
template <int N>
__device__ __forceinline__ void lds_run(const uint8_t* p, uint32_t phase, uint32_t (&o)[N]) {
  const uint8_t* a = p - phase;
  uint32_t w[N + 1];
#pragma unroll
  for (int k = 0; k <= N; ++k) w[k] = lds4(a + 4 * k);
#pragma unroll
  for (int k = 0; k < N; ++k) o[k] = __builtin_amdgcn_alignbyte(w[k + 1], w[k], phase);
}

// The streamed lane parts take the lane's x as XL limb planes of XN / 4 dwords (xq), the
// stored scale of each of its 32-column blocks (xsc) and the fp32 sums of each 16 columns
// (xs), as staged by limb_digits / limb_scale.

// Q6_K lane part: quarter g = 2n + hi of superblock s: columns 128n + 64hi + l (l < 64).
// Column 128n + 64hi + l for l < 32 takes the low (hi = 0) or high (hi = 1) nibble of
// low-bit byte 64n + l and bits 4hi..4hi+1 of high-bit byte 32n + l; for l >= 32 the
// nibble of byte 64n + l and bits 4hi+2..4hi+3 of high-bit byte 32n + l - 32.  Scale of
// columns 16j.. of the quarter: int8 at 192 + 8n + 4hi + j (j = 0..3); w = d sc (q - 32),
// summed per 16 columns as d sc (s sum q x~ - 32 sum x).  The four codes of a dword are
// the nibbles (shifted down by 4hi) with the top bits rotated into bits 4..5 of each byte.
// A superblock at an odd index sits 2 bytes past a 4-byte boundary in the ring; its fields
// are realigned per lane.
struct Q6K_S {
  static constexpr int FMT = FMT_Q6_K, BB = 210, K = 1;
  static __device__ __forceinline__ float dot(const uint8_t* slot, int lane, const uint32_t (&xq)[XL][16],
                                              const float (&xsc)[2], const float (&xs)[4]) {
    const int s = lane >> 2, g = lane & 3, n = g >> 1, hi = g & 1;
    const uint8_t* p = slot + s * 210;
    const uint32_t ph = (uint32_t)(s & 1) * 2u;
    uint32_t S[1], D[1];
    // high-bit bytes: the nine aligned words around the eight the lane needs; a lane whose
    // rotation moves bits left (hi = 0) at phase 0 takes them one word earlier, so that for
    // every lane one funnel shift of words k + 1, k by (8 phase + rotation) mod 32 realigns and
    // rotates at once (the bits that come from the other word are masked off)
    uint32_t Hw[9];
    {
      const uint8_t* hp = p + 128 + 32 * n - ph - ((ph == 0 && hi == 0) ? 4 : 0);
#pragma unroll
      for (int k = 0; k <= 8; ++k) Hw[k] = lds4(hp + 4 * k);
    }
    lds_run<1>(p + 192 + 8 * n + 4 * hi, ph, S);
    lds_run<1>(p + 208, ph, D);
    const uint32_t m0f = vreg(0x0F0F0F0Fu), m30 = vreg(0x30303030u);
    const uint32_t sl = 4u * (uint32_t)hi;
    int dg[4][XL];  // per 16 columns
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int l = 0; l < XL; ++l) dg[j][l] = 0;
    // the low-bit bytes' nibble is taken from the two aligned words around each word with one
    // funnel shift by 8 phase + 4 hi, which realigns and shifts at once
    const uint32_t lsh = 8u * ph + sl;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t Lw[9];
      const uint8_t* lp = p + 64 * n + 32 * half - ph;
#pragma unroll
      for (int k = 0; k <= 8; ++k) Lw[k] = lds4(lp + 4 * k);
      const uint32_t rot = (sl + 2u * (uint32_t)half + 28u) & 31u;  // top bits 4hi + 2half -> bit 4
      const uint32_t hsh = (8u * ph + rot) & 31u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t lo = __builtin_amdgcn_alignbit(Lw[k + 1], Lw[k], lsh) & m0f;
        const uint32_t code = and_or(__builtin_amdgcn_alignbit(Hw[k + 1], Hw[k], hsh), m30, lo);
        int(&d)[XL] = dg[2 * half + (k >> 2)];
#pragma unroll
        for (int l = 0; l < XL; ++l) d[l] = (k & 3) == 0 ? sdot4_0(code, xq[l][8 * half + k]) : sdot4(code, xq[l][8 * half + k], d[l]);
      }
    }
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = (float)(int8_t)((S[0] >> (8 * j)) & 0xFFu);
      r += sc * (xsc[j >> 1] * limb_sum(dg[j]) - 32.f * xs[j]);
    }
    return h2f(D[0]) * r;
  }
};

// Q8_0 lane part: block l: fp16 d, then 32 int8 q; w = d q.
struct Q80_S {
  static constexpr int FMT = FMT_Q8_0, BB = 34, K = 0;
  static __device__ __forceinline__ float dot(const uint8_t* slot, int lane, const uint32_t (&xq)[XL][8],
                                              const float (&xsc)[1], const float (&xs)[2]) {
    (void)xs;
    const uint8_t* p = slot + lane * 34;
    const uint32_t pd = (uint32_t)(lane & 1) * 2u;  // 34 lane mod 4
    uint32_t Q[8], D[1];
    lds_run<8>(p + 2, 2u - pd, Q);
    lds_run<1>(p, pd, D);
    int d[XL];
#pragma unroll
    for (int l = 0; l < XL; ++l) d[l] = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int l = 0; l < XL; ++l) d[l] = sdot4(Q[k], xq[l][k], d[l]);
    return h2f(D[0]) * (xsc[0] * limb_sum(d));
  }
};

// Q4_0 lane part: block l: fp16 d, then 16 bytes; column i < 16 is the low nibble of
// byte i, column 16 + i the high nibble; w = d (q - 8).
struct Q40_S {
  static constexpr int FMT = FMT_Q4_0, BB = 18, K = 0;
  static __device__ __forceinline__ float dot(const uint8_t* slot, int lane, const uint32_t (&xq)[XL][8],
                                              const float (&xsc)[1], const float (&xs)[2]) {
    const uint8_t* p = slot + lane * 18;
    const uint32_t pd = (uint32_t)(lane & 1) * 2u;  // 18 lane mod 4
    uint32_t Q[4], D[1];
    lds_run<4>(p + 2, 2u - pd, Q);
    lds_run<1>(p, pd, D);
    const uint32_t m0f = vreg(0x0F0F0F0Fu);
    int d[XL];
#pragma unroll
    for (int l = 0; l < XL; ++l) d[l] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = Q[k] & m0f, hi = (Q[k] >> 4) & m0f;
#pragma unroll
      for (int l = 0; l < XL; ++l) {
        d[l] = sdot4(lo, xq[l][k], d[l]);
        d[l] = sdot4(hi, xq[l][4 + k], d[l]);
      }
    }
    return h2f(D[0]) * (xsc[0] * limb_sum(d) - 8.f * (xs[0] + xs[1]));
  }
};

struct StreamArgs {
  GemvArgs a;
  int tstart[3];   // first task of each segment
  int tasks;       // tasks of the launch (SWIGLU: 2 per row, gate then up)
  int tpw;         // tasks per workgroup (even)
  int ns;          // column slices
  int rsub;        // waves per slice
  int xring;       // 1: the x slice is staged through the slice's rings (they hold a whole slice);
                   // 2: the x slice and the gain slice (they hold both)
};

// Per-wave constants of the launch's segments (one for STORE / RESID / LOGITS, gate and
// up for SWIGLU, q / k / v for QKV), kept in registers across the task loop.
template <int EPI>
struct SegCache {
  static constexpr int NS = (EPI == EPI_SWIGLU) ? 2 : (EPI == EPI_QKV) ? 3 : 1;
  const uint8_t* base[NS];  // this wave's slice of row 0
  int64_t rb[NS];           // row bytes
  int last[NS];             // index of the slice's last 16-byte piece
  int fmt[NS];
  int ts1, ts2;             // first task of segments 1 and 2 (QKV)
};

template <int KF, int EPI>
__device__ __forceinline__ SegCache<EPI> seg_cache(const StreamArgs& sa, int sl) {
  SegCache<EPI> c;
  constexpr int per_slice = KF ? (ST_SLICE_COLS_K / 256) : (ST_SLICE_COLS_B / 32);
  const int b0 = sl * per_slice;
  const int nb = min(per_slice, sa.a.cols / (KF ? 256 : 32) - b0);
#pragma unroll
  for (int i = 0; i < SegCache<EPI>::NS; ++i) {
    const GemvSeg& sg = sa.a.seg[i];
    const int bb = block_bytes(sg.fmt);
    c.base[i] = sg.w + (size_t)b0 * bb;
    c.rb[i] = sg.row_bytes;
    c.last[i] = ((nb * bb) >> 4) - 1;
    c.fmt[i] = sg.fmt;
  }
  c.ts1 = sa.tstart[1];
  c.ts2 = sa.tstart[2];
  return c;
}

// Segment and row of task t.
template <int EPI>
__device__ __forceinline__ void st_task(const SegCache<EPI>& c, int t, int& seg, int& row) {
  if constexpr (EPI == EPI_SWIGLU) {
    seg = t & 1;
    row = t >> 1;
  } else if constexpr (EPI == EPI_QKV) {
    seg = t >= c.ts2 ? 2 : t >= c.ts1 ? 1 : 0;
    row = t - (seg == 2 ? c.ts2 : seg == 1 ? c.ts1 : 0);
  } else {
    seg = 0;
    row = t;
  }
}

template <int EPI, typename T>
__device__ __forceinline__ T seg_pick(const T (&v)[SegCache<EPI>::NS], int seg) {
  if constexpr (SegCache<EPI>::NS == 1) return v[0];
  else if constexpr (SegCache<EPI>::NS == 2) return seg ? v[1] : v[0];
  else return seg == 2 ? v[2] : seg == 1 ? v[1] : v[0];
}

// Issue the NI transfers of task t's slice bytes into a ring slot.  Lanes past the slice's
// last 16-byte piece re-read that piece, so every task issues exactly NI instructions.
template <int EPI, int NI>
__device__ __forceinline__ void st_issue(const SegCache<EPI>& c, int t, int lane, uint8_t* slot) {
  int seg, row;
  st_task<EPI>(c, t, seg, row);
  const uint8_t* src = seg_pick<EPI>(c.base, seg) + (size_t)row * seg_pick<EPI>(c.rb, seg);
  const int last = seg_pick<EPI>(c.last, seg);
#pragma unroll
  for (int i = 0; i < NI; ++i) dma16(src + 16 * min(64 * i + lane, last), slot + 1024 * i);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Sum over each row of 16 lanes, left in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}

// A lane's XN floats (its own columns, XN / 4 float4 from float4 lane XN / 4 of the vector)
// from the slice's rings, where float4 f of a vector sits in slot base + s(f), s(f) = f with
// its position in its block of 16 rotated by the block index (so that the 16-byte reads of
// 16 consecutive lanes fall on distinct banks); slot s is in the ring of the slice's wave
// s / (RB / 16), at byte 16 (s mod (RB / 16)).
template <int XN, int RB>
__device__ __forceinline__ void x_from_rings(float (&x)[XN], const uint8_t* lds0, int base, int lane, int sl, int ns) {
#pragma unroll
  for (int q = 0; q < XN / 4; ++q) {
    const int f = lane * (XN / 4) + q;
    const int sidx = base + ((f & ~15) | ((f + (f >> 4)) & 15));
    const int so = sidx / (RB / 16);
    const float4 v = *reinterpret_cast<const float4*>(lds0 + (size_t)(so * ns + sl) * RB + (sidx % (RB / 16)) * 16);
    x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
  }
}

template <int KF, int EPI, int D, int NI>
__global__ __launch_bounds__(ST_MAX_WAVES * 64) void gemv_stream_kernel(const StreamArgs sa) {
  constexpr int XN = KF ? 64 : 32;   // x values per lane
  constexpr int XG = KF ? 4 : 2;     // 16-column sums per lane
  constexpr int SLOT = 1024 * NI;
  extern __shared__ float4 smem4[];
  const GemvArgs& a = sa.a;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (int)(blockDim.x >> 6);
  const int sl = wave % sa.ns, sub = wave / sa.ns;
  const SegCache<EPI> sc = seg_cache<KF, EPI>(sa, sl);
  uint8_t* ring = reinterpret_cast<uint8_t*>(smem4) + (size_t)wave * D * SLOT;
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(smem4) + (size_t)nw * D * SLOT);
  __shared__ float ssq[ST_MAX_WAVES];
  __shared__ float2 rope[64];
  __shared__ unsigned long long wbest[ST_MAX_WAVES];
  if constexpr (EPI == EPI_QKV) {
    if (threadIdx.x < 64) rope[threadIdx.x] = rope_cs(a.rope_theta, a.pos, threadIdx.x, 128);
  }
  const int t0 = (int)blockIdx.x * sa.tpw, t1 = min(sa.tasks, t0 + sa.tpw);
  // The waves of a slice share its tasks: each starts with D fixed ones (t0 + sub + d rsub)
  // and then takes the next untaken task of the slice from a counter in LDS, so that waves
  // slowed by their place in the memory queues do fewer tasks instead of finishing last.
  __shared__ int next_task[ST_MAX_WAVES];
  if ((int)threadIdx.x < sa.ns) next_task[threadIdx.x] = t0 + D * sa.rsub;
  __syncthreads();

  // ---- x slice into registers, issued first so that it arrives first
  constexpr int SC = KF ? ST_SLICE_COLS_K : ST_SLICE_COLS_B;  // columns of a slice
  constexpr int RB = D * SLOT;                                 // ring bytes of a wave
  const int c0 = sl * SC + XN * lane;
  const bool xvalid = c0 < a.cols;
  float x[XN];
  if (sa.xring) {
    // A lane's columns are XN consecutive floats, so lane-contiguous loads of them touch 64
    // lines per instruction and occupy the CU's load path ~16 times longer than loads of
    // whole lines; the later waves of a workgroup then wait microseconds for x.  Instead
    // the slice goes through the slice's rings first (before any weight transfer): each
    // wave moves its share with the global->LDS path, 1 KiB of whole lines per instruction,
    // in a swizzled order (float4 f of a block of 16 at position (f + block) mod 16), so
    // that the lanes' 16-byte reads of their own columns below meet no bank conflicts.
    // With a gain (xring 2) its slice follows x's in the rings, and the norm is applied
    // below before the rings are refilled.
    constexpr int NF = SC / 4;                   // float4 of a slice (a multiple of 64)
    const int lim = (a.cols - sl * SC) / 4;      // valid float4 of this slice
    const int nslots = sa.xring == 2 ? 2 * NF : NF;
#pragma unroll
    for (int k = 0; k < RB / 1024; ++k) {
      if (sub * (RB / 16) + 64 * k < nslots) {   // wave-uniform
        const int sidx = sub * (RB / 16) + 64 * k + lane;  // slot of this lane's float4
        const int vec = sidx >= NF ? 1 : 0;      // 0: x, 1: gain (wave-uniform: NF % 64 == 0)
        const int sv = sidx - vec * NF;
        const int blk = sv >> 4;
        int f = 16 * blk + (((sv & 15) - blk) & 15);
        f = f < lim ? f : 0;                     // past the last column: a valid address, unused
        dma16c((vec ? a.gain : a.x) + (size_t)sl * SC + 4 * f, ring + 1024 * k);
      }
    }
    wait_vm<0>();
    __syncthreads();
    x_from_rings<XN, RB>(x, reinterpret_cast<const uint8_t*>(smem4), 0, lane, sl, sa.ns);
    if (sa.xring == 2) {
      // the norm's scale from the sum of squares over all slices, then the gain from the rings
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < XN; ++i) q += x[i] * x[i];
      q = wave_sum(xvalid ? q : 0.f);
      if (sub == 0 && lane == 0) ssq[sl] = q;
      __syncthreads();
      float tot = 0.f;
      for (int i = 0; i < sa.ns; ++i) tot += ssq[i];
      const float scale = 1.0f / sqrtf(tot / (float)a.cols + a.eps);
      float g[XN];
      x_from_rings<XN, RB>(g, reinterpret_cast<const uint8_t*>(smem4), NF, lane, sl, sa.ns);
#pragma unroll
      for (int i = 0; i < XN; ++i) x[i] = x[i] * scale * g[i];
    }
    __syncthreads();  // every ring read before the weight transfers below refill it
  } else {
    const float4* xp = reinterpret_cast<const float4*>(a.x + (xvalid ? c0 : 0));
#pragma unroll
    for (int i = 0; i < XN / 4; ++i) {
      const float4 v = xp[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- the first D tasks of this wave in flight (every wave has a slice and a share of tasks)
  int tslot[D];  // the task in each ring slot (t1 or more: none)
#pragma unroll
  for (int d = 0; d < D; ++d) {
    tslot[d] = t0 + sub + d * sa.rsub;
    st_issue<EPI, NI>(sc, min(tslot[d], t1 - 1), lane, ring + d * SLOT);
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- RMSNorm prologue: scale from the sum of squares over all slices (unless done above)
  if (a.gain && sa.xring != 2) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < XN; ++i) q += x[i] * x[i];
    q = wave_sum(xvalid ? q : 0.f);
    if (sub == 0 && lane == 0) ssq[sl] = q;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < sa.ns; ++i) tot += ssq[i];
    const float scale = 1.0f / sqrtf(tot / (float)a.cols + a.eps);
    const float4* gp = reinterpret_cast<const float4*>(a.gain + (xvalid ? c0 : 0));
#pragma unroll
    for (int i = 0; i < XN / 4; ++i) {
      const float4 gg = gp[i];
      x[4 * i] = x[4 * i] * scale * gg.x;
      x[4 * i + 1] = x[4 * i + 1] * scale * gg.y;
      x[4 * i + 2] = x[4 * i + 2] * scale * gg.z;
      x[4 * i + 3] = x[4 * i + 3] * scale * gg.w;
    }
  }
  float xs[XG];
#pragma unroll
  for (int j = 0; j < XG; ++j) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) t += x[16 * j + i] + x[16 * j + i + 1];
    xs[j] = t;
  }
  // the lane's columns are whole 32-column blocks: their limbs and scales, as staged for
  // the register path
  uint32_t xq[XL][XN / 4];
  float xsc[XN / 32];
#pragma unroll
  for (int b = 0; b < XN / 32; ++b) {
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) mb = max(mb, __float_as_uint(x[32 * b + i]) & 0x7FFFFFFFu);
    float k;
    limb_scale(mb, xsc[b], k);
#pragma unroll
    for (int i = 0; i < 8; ++i) limb_digits(&x[32 * b + 4 * i], k, xq, 8 * b + i);
  }

  // ---- the wave's tasks, in the order its ring slots were filled; every refill issues the
  // same transfers (past the last task it re-reads the last row), so the wait is static
  // (the ring is unrolled, so that the slots' tasks stay in registers)
  for (bool more = true; more;) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = tslot[d];
      if (t >= t1) {  // tasks are taken in increasing order: the later slots hold none either
        more = false;
        break;
      }
      uint8_t* slot = ring + d * SLOT;
      wait_vm<NI * (D - 1)>();
      int seg, row;
      st_task<EPI>(sc, t, seg, row);
      float v = 0.f;
      if (xvalid) {
        const int fmt = seg_pick<EPI>(sc.fmt, seg);
        if constexpr (KF) {
          v = Q6K_S::dot(slot, lane, xq, xsc, xs);  // the launcher sends Q4_K to the register path
        } else {
          if (fmt == FMT_Q8_0) v = Q80_S::dot(slot, lane, xq, xsc, xs);
          else v = Q40_S::dot(slot, lane, xq, xsc, xs);
        }
      }
      // the slot has been read: refill it with the slice's next untaken task
      int tn = 0;
      if (lane == 0) tn = atomicAdd(&next_task[sl], 1);
      tn = __builtin_amdgcn_readfirstlane(tn);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      st_issue<EPI, NI>(sc, min(tn, t1 - 1), lane, slot);
      tslot[d] = tn;
      v = row16_sum(v);
      if ((lane & 15) == 0) part[(((t - t0) * sa.ns + sl) << 2) + (lane >> 4)] = v;
    }
  }
  wait_vm<0>();
  __syncthreads();

  // ---- epilogue: one thread per task (per pair for SWIGLU and QKV)
  unsigned long long best = 0;
  const int nt = t1 - t0;
  auto total = [&](int i) {
    const float4* q = reinterpret_cast<const float4*>(part) + i * sa.ns;
    float v = 0.f;
    for (int j = 0; j < sa.ns; ++j) {
      const float4 f = q[j];
      v += (f.x + f.y) + (f.z + f.w);
    }
    return v;
  };
  if constexpr (EPI == EPI_STORE || EPI == EPI_LOGITS || EPI == EPI_RESID) {
    for (int i = threadIdx.x; i < nt; i += blockDim.x) {
      const int r = t0 + i;
      const float v = total(i);
      if constexpr (EPI == EPI_RESID) {
        const float o = a.resid[r] + v;
        a.y[r] = o;
        if (a.y2) a.y2[r] = o;
      } else {
        a.y[r] = v;
      }
      if constexpr (EPI == EPI_LOGITS) {
        const unsigned long long key = logit_key(v, r);
        best = key > best ? key : best;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int i = 2 * threadIdx.x; i < nt; i += 2 * blockDim.x) a.y[(t0 + i) >> 1] = silu_mul(total(i), total(i + 1));
  } else if constexpr (EPI == EPI_QKV) {
    constexpr int HD = 128;
    for (int i = 2 * threadIdx.x; i < nt; i += 2 * blockDim.x) {
      int seg, r;
      st_task<EPI>(sc, t0 + i, seg, r);
      const float y0 = total(i), y1 = total(i + 1);
      const int head = r / HD, dd = r % HD;
      if (seg < 2) {
        const float2 c = rope[dd >> 1];
        const float r0 = y0 * c.x - y1 * c.y;
        const float r1 = y0 * c.y + y1 * c.x;
        if (seg == 0) {
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
  if constexpr (EPI == EPI_LOGITS) {
    // one atomic per workgroup
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long b = 0;
      for (int w = 0; w < nw; ++w) b = wbest[w] > b ? wbest[w] : b;
      if (b) atomicMax(a.amax, b);
    }
  }
}

// ------------------------------------------------------------------ host side

// Host-side state is set up once, with C++ static initialisation (thread-safe), or kept in
// one atomic word, so that concurrent calls from several host threads cannot race on it.

// compute units of the device current at the first call (one MI355X: 256)
static int num_cu() {
  static const int n_cu = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      return n;
    return 256;
  }();
  return n_cu;
}

constexpr size_t GEMV_LDS_MAX = 160 * 1024 - 2048;  // dynamic LDS budget of the register path (static LDS on top)

// limb planes (quantized formats), fp32 x (unquantized formats), scales per 32 columns, sums
// per 16 columns, 16 floats of reduction space
static size_t lds_for(int cols, int inst) {
  return (mask_has_q(inst) ? (size_t)XL * xq_plane(cols) : 0) + (mask_has_f(inst) ? sizeof(float) * (size_t)cols : 0) +
         sizeof(float) * (size_t)((cols >> 5) + (cols >> 4) + 16);
}

// The kernel instantiation a launch's format mask selects (launch_mask; the fixed q/k/v format
// variants stage what their general masks stage).
static int inst_mask(int m) {
  switch (m) {
    case 1 << FMT_Q8_0: case 1 << FMT_Q4_0: case 1 << FMT_Q4_K: case 1 << FMT_Q6_K: case 1 << FMT_Q5_K:
    case 1 << FMT_F16: case 1 << FMT_F32: case 1 << FMT_Q4_KT: case 1 << FMT_Q8_0T: case 1 << FMT_Q5_KT:
    case (1 << FMT_Q5_KT) | (1 << FMT_Q6_K):
    case (1 << FMT_Q5_K) | (1 << FMT_Q6_K): case (1 << FMT_Q4_K) | (1 << FMT_Q6_K): case (1 << FMT_Q4_KT) | (1 << FMT_Q6_K):
      return m;
    default:
      return (1 << FMT_COUNT) - 1;
  }
}

// Formats whose single-format instantiations also come with one row per work item.
static bool one_row_mask(int m) {
  switch (m) {
    case 1 << FMT_Q8_0: case 1 << FMT_Q4_0: case 1 << FMT_Q4_K: case 1 << FMT_Q6_K: case 1 << FMT_Q5_K:
    case 1 << FMT_F16: case 1 << FMT_F32: case 1 << FMT_Q4_KT: case 1 << FMT_Q8_0T: case 1 << FMT_Q5_KT:
      return true;
    default:
      return false;
  }
}

GemvPlan gemv_plan(int epi, int cols, int fmt_mask, int rows) {
  GemvPlan p;
  p.rows_per_wave = (epi == EPI_SWIGLU) ? 1 : (epi == EPI_QKV) ? 2 : NT_GEMV_ROWS;
  // a short matrix (at most half as many rows as the chip has wave slots, 16 per CU) would
  // leave most waves idle with row pairs: one row per work item then (measured: Q6_K
  // 1024 x 8192 9.6 -> 6.8 us, Q4_K 1024 x 8192 5.9 -> 5.0 us; at 4096 rows pairs are faster)
  if (p.rows_per_wave == 2 && epi != EPI_QKV && rows > 0 && one_row_mask(fmt_mask) && rows <= 8 * num_cu())
    p.rows_per_wave = 1;
  p.lds_bytes = lds_for(cols, inst_mask(fmt_mask));
  // one copy of x per workgroup: when only one fits in a CU's LDS, make it 16 waves
  p.waves = p.lds_bytes > 80 * 1024 ? 16 : 8;
  return p;
}

int gemv_groups(const GemvPlan& p, int rows) { return (rows + p.rows_per_wave - 1) / p.rows_per_wave; }

template <int FMTMASK, int NW, int EPI, int R>
static hipError_t launch_one(const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  auto kern = gemv_kernel<FMTMASK, R, NW, EPI>;
  // the dynamic LDS limit, raised once to the whole budget (each launch passes its own size)
  static const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMV_LDS_MAX);
  if (raised != hipSuccess) return raised;
  // the plan must hold what this instantiation stages
  if (plan.lds_bytes > GEMV_LDS_MAX || plan.lds_bytes < lds_for(a.cols, FMTMASK)) return hipErrorInvalidValue;
  // resident workgroups per CU at this LDS size, cached per instantiation as (LDS bytes << 8 | count)
  static std::atomic<uint64_t> cache{0};
  const uint64_t c = cache.load(std::memory_order_relaxed);
  int per_cu = (int)(c & 0xFF);
  if (per_cu == 0 || (c >> 8) != (uint64_t)plan.lds_bytes) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NW * 64, plan.lds_bytes);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? (n < 255 ? n : 255) : 1;
    if (NT_GEMV_WG_PER_CU_MAX > 0 && per_cu > NT_GEMV_WG_PER_CU_MAX) per_cu = NT_GEMV_WG_PER_CU_MAX;
    cache.store(((uint64_t)plan.lds_bytes << 8) | (uint64_t)per_cu, std::memory_order_relaxed);
  }
  // as many resident waves as the chip holds, but no idle workgroups
  const int grid = max(1, min((n_groups + NW - 1) / NW, per_cu * num_cu()));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), plan.lds_bytes, s, a);
  return hipGetLastError();
}

template <int FMTMASK, int EPI, int R>
static hipError_t launch_nw_r(const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  switch (plan.waves) {
    case 8: return launch_one<FMTMASK, 8, EPI, R>(plan, n_groups, a, s);
    case 16: return launch_one<FMTMASK, 16, EPI, R>(plan, n_groups, a, s);
    default: return hipErrorInvalidConfiguration;
  }
}

// rows per work item as the plan says: the epilogue's own count, or one for the single-format
// instantiations of the plain, residual and logits epilogues
template <int FMTMASK, int EPI>
static hipError_t launch_nw(const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  constexpr int R = GEMV_ROWS<EPI>;
  constexpr int FM = FMTMASK & ~FMT_NTL;
  if constexpr (R == 2 && EPI != EPI_QKV && (FM & (FM - 1)) == 0 && FM < (1 << FMT_COUNT)) {
    if (plan.rows_per_wave == 1) return launch_nw_r<FMTMASK, EPI, 1>(plan, n_groups, a, s);
  }
  if (plan.rows_per_wave != R) return hipErrorInvalidConfiguration;
  return launch_nw_r<FMTMASK, EPI, R>(plan, n_groups, a, s);
}

template <int EPI>
static hipError_t launch_mask(int fmt_mask, const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  switch (fmt_mask) {
    case 1 << FMT_Q8_0: return launch_nw<1 << FMT_Q8_0, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q4_0: return launch_nw<1 << FMT_Q4_0, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q4_K: return launch_nw<1 << FMT_Q4_K, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q6_K: return launch_nw<1 << FMT_Q6_K, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q5_K: return launch_nw<1 << FMT_Q5_K, EPI>(plan, n_groups, a, s);
    case 1 << FMT_F16: return launch_nw<1 << FMT_F16, EPI>(plan, n_groups, a, s);
    case 1 << FMT_F32: return launch_nw<1 << FMT_F32, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q5_K) | (1 << FMT_Q6_K):
      if constexpr (EPI == EPI_QKV) {
        if (a.nseg == 3 && a.seg[0].fmt == FMT_Q5_K && a.seg[1].fmt == FMT_Q5_K && a.seg[2].fmt == FMT_Q6_K)
          return launch_nw<FMTS_Q5K_Q5K_Q6K, EPI>(plan, n_groups, a, s);
      }
      return launch_nw<(1 << FMT_Q5_K) | (1 << FMT_Q6_K), EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q4_K) | (1 << FMT_Q6_K):
      if constexpr (EPI == EPI_QKV) {
        if (a.nseg == 3 && a.seg[0].fmt == FMT_Q4_K && a.seg[1].fmt == FMT_Q4_K && a.seg[2].fmt == FMT_Q6_K)
          return launch_nw<FMTS_Q4K_Q4K_Q6K, EPI>(plan, n_groups, a, s);
      }
      return launch_nw<(1 << FMT_Q4_K) | (1 << FMT_Q6_K), EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q4_KT: return launch_nw<1 << FMT_Q4_KT, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q4_KT) | FMT_NTL: return launch_nw<(1 << FMT_Q4_KT) | FMT_NTL, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q8_0T: return launch_nw<1 << FMT_Q8_0T, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q8_0T) | FMT_NTL: return launch_nw<(1 << FMT_Q8_0T) | FMT_NTL, EPI>(plan, n_groups, a, s);
    case 1 << FMT_Q5_KT: return launch_nw<1 << FMT_Q5_KT, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q5_KT) | FMT_NTL: return launch_nw<(1 << FMT_Q5_KT) | FMT_NTL, EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q5_KT) | (1 << FMT_Q6_K): return launch_nw<(1 << FMT_Q5_KT) | (1 << FMT_Q6_K), EPI>(plan, n_groups, a, s);
    case (1 << FMT_Q4_KT) | (1 << FMT_Q6_K):
      if constexpr (EPI == EPI_QKV) {
        if (a.nseg == 3 && a.seg[0].fmt == FMT_Q4_KT && a.seg[1].fmt == FMT_Q4_KT && a.seg[2].fmt == FMT_Q6_K)
          return launch_nw<FMTS_Q4KT_Q4KT_Q6K, EPI>(plan, n_groups, a, s);
      }
      return launch_nw<(1 << FMT_Q4_KT) | (1 << FMT_Q6_K), EPI>(plan, n_groups, a, s);
    default: return launch_nw<(1 << FMT_COUNT) - 1, EPI>(plan, n_groups, a, s);
  }
}

// ---- streamed path
static bool st_family(int fmt) { return fmt == FMT_Q4_K || fmt == FMT_Q6_K; }
// launches with fewer weights take the register path (see gemv_stream_launch)
static std::atomic<int64_t> g_st_min_weights{100000000};

int64_t gemv_set_stream_min_weights(int64_t w) {
  return w < 0 ? g_st_min_weights.load(std::memory_order_relaxed) : g_st_min_weights.exchange(w, std::memory_order_relaxed);
}

constexpr size_t ST_LDS_MAX = 160 * 1024 - 2048;  // dynamic LDS budget (static LDS on top)

template <int KF, int EPI, int D, int NI>
static hipError_t st_launch(const StreamArgs& sa, int grid, int nw, size_t lds, hipStream_t s) {
  auto kern = gemv_stream_kernel<KF, EPI, D, NI>;
  static const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)ST_LDS_MAX);
  if (raised != hipSuccess) return raised;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(nw * 64), lds, s, sa);
  return hipGetLastError();
}

// Ring configurations: transfers per task NI (slot = NI KiB) and ring depth D.
template <int EPI>
static hipError_t st_dispatch(bool kf, int ni, int d, const StreamArgs& sa, int grid, int nw, size_t lds, hipStream_t s) {
  if (kf) {
    if (ni == 3) return d == 3 ? st_launch<1, EPI, 3, 3>(sa, grid, nw, lds, s) : st_launch<1, EPI, 2, 3>(sa, grid, nw, lds, s);
    return st_launch<1, EPI, 2, 4>(sa, grid, nw, lds, s);
  }
  if (ni == 2) return d == 3 ? st_launch<0, EPI, 3, 2>(sa, grid, nw, lds, s) : st_launch<0, EPI, 2, 2>(sa, grid, nw, lds, s);
  return d == 3 ? st_launch<0, EPI, 3, 3>(sa, grid, nw, lds, s) : st_launch<0, EPI, 2, 3>(sa, grid, nw, lds, s);
}

// Work items that each busy wave of the register path runs one after another for this launch
// (row groups per wave, the chip holding 16 waves per CU, times steps per row; 0 for the
// formats the streamed path does not take).
static int reg_depth(int fmt, int cols, int n_groups) {
  int steps;
  switch (fmt) {
    case FMT_Q8_0: case FMT_Q4_0: steps = Q8_0F::steps(cols); break;
    case FMT_Q6_K: steps = Q6_KF::steps(cols); break;
    default: return 0;
  }
  const int waves = 16 * num_cu();
  return (n_groups + waves - 1) / waves * steps;
}

// Launch the streamed path if the shape allows it (rows and x 16-byte aligned, one format
// family).  Returns hipErrorNotSupported, with nothing launched, if it does not.
static hipError_t gemv_stream_launch(int epi, const GemvArgs& a, int n_groups, hipStream_t s) {
  const int nseg = (epi == EPI_SWIGLU) ? 2 : a.nseg;
  // the kernel's segment layout: one matrix, gate + up, or q + k + v
  if (nseg != (epi == EPI_SWIGLU ? 2 : epi == EPI_QKV ? 3 : 1)) return hipErrorNotSupported;
  const bool kf = st_family(a.seg[0].fmt);
  // The streamed path pays more per launch than the register path (its rings fill before the
  // first product), which only its higher rate on large launches earns back: below 10^8
  // weights per launch the register path is as fast or faster (measured, register vs
  // streamed: Q8_0 4096 x 4096 6.7 vs 9.4 us, Q4_0 4096 x 8192 7.5 vs 10.0 us; within a few
  // percent near the threshold: Q6_K 8192 x 8192 19.2 vs 18.6 us; above it Q6_K 8192 x 28672
  // 57 vs 44.5 us), except where the register path's waves would each run 7 or more items in a row (long
  // rows over few row groups: the streamed path splits a row's columns over several waves).
  // From an eighth of the threshold such deep launches stream too (measured, register vs
  // streamed: Q8_0 4096 x 14336 (depth 8) 22.7 vs 16.4 us, 1024 x 28672 (14) 22.2 vs 13.0 us,
  // 28672 x 1024 (8) 12.7 vs 11.9 us, 2048 x 14336 (8) 11.8 vs 11.6 us; Q6_K 4096 x 28672 (14)
  // 44.2 vs 26.8 us; at depth 4: Q8_0 4096 x 8192 10.9 vs 12.4 us, Q4_0 8192 x 8192 13.0 vs
  // 13.3 us).  A threshold of 0 streams every launch the formats allow.
  int64_t weights = 0;
  for (int i = 0; i < nseg; ++i) weights += (int64_t)a.seg[i].rows * a.cols;
  const int64_t t = g_st_min_weights.load(std::memory_order_relaxed);
  if (weights < t && !(weights >= t / 8 && reg_depth(a.seg[0].fmt, a.cols, n_groups) >= 7)) return hipErrorNotSupported;
  for (int i = 0; i < nseg; ++i) {
    const GemvSeg& g = a.seg[i];
    if (st_family(g.fmt) != kf) return hipErrorNotSupported;
    // Q4_K measured faster on the register path (also with integer dot products here:
    // 64.7 vs 49.9 us for the 70B gate/up pair); Q5_K, its 5-bit sibling, and the tiled
    // layouts Q4_KT and Q8_0T have only that path
    if (g.fmt == FMT_Q4_K || g.fmt == FMT_Q4_KT || g.fmt == FMT_Q8_0T || g.fmt == FMT_Q5_K || g.fmt == FMT_Q5_KT ||
        is_float_fmt(g.fmt))
      return hipErrorNotSupported;
    if ((reinterpret_cast<uintptr_t>(g.w) & 15) || (g.row_bytes & 15) || g.rows <= 0) return hipErrorNotSupported;
  }
  if ((reinterpret_cast<uintptr_t>(a.x) & 15) || (a.gain && (reinterpret_cast<uintptr_t>(a.gain) & 15)))
    return hipErrorNotSupported;
  const int slice_cols = kf ? ST_SLICE_COLS_K : ST_SLICE_COLS_B;
  if (a.cols % (kf ? 256 : 32)) return hipErrorNotSupported;
  StreamArgs sa;
  sa.a = a;
  sa.ns = (a.cols + slice_cols - 1) / slice_cols;
  if (sa.ns > ST_MAX_WAVES) return hipErrorNotSupported;
  int slot = 0;
  for (int i = 0; i < nseg; ++i) {
    const int per_slice = kf ? slice_cols / 256 : slice_cols / 32;
    const int nblk = a.cols / (kf ? 256 : 32);
    // + 16: the realigning LDS reads of the last block may run up to 6 bytes past it
    const int bytes = min(per_slice, nblk) * block_bytes(a.seg[i].fmt) + 16;
    slot = max(slot, (bytes + 1023) / 1024 * 1024);
  }
  // the instantiated slot sizes: 3 or 4 KiB (superblock formats), 2 or 3 KiB (block formats)
  int ni = slot / 1024;
  if (kf) ni = ni <= 3 ? 3 : ni;
  else ni = ni <= 2 ? 2 : ni;
  if (ni > (kf ? 4 : 3)) return hipErrorNotSupported;
  int tasks = 0;
  if (epi == EPI_SWIGLU) {
    if (a.seg[1].rows != a.seg[0].rows) return hipErrorNotSupported;
    tasks = 2 * a.seg[0].rows;
    sa.tstart[0] = 0; sa.tstart[1] = 0; sa.tstart[2] = 0;
  } else {
    for (int i = 0; i < nseg; ++i) {
      sa.tstart[i] = tasks;
      if ((epi == EPI_QKV) && (a.seg[i].rows & 1)) return hipErrorNotSupported;
      tasks += a.seg[i].rows;
    }
    for (int i = nseg; i < 3; ++i) sa.tstart[i] = tasks;
  }
  sa.tasks = tasks;
  const int ncu = num_cu();
  int tpw = (tasks + ncu - 1) / ncu;
  tpw = max(2, (tpw + 1) & ~1);
  sa.tpw = tpw;
  const int grid = (tasks + tpw - 1) / tpw;
  const size_t part = (size_t)tpw * sa.ns * 4 * sizeof(float);
  const size_t slot_bytes = (size_t)ni * 1024;
  int rsub = max(1, ST_MAX_WAVES / sa.ns);
  int d = 3;
  for (;;) {
    const size_t nw = (size_t)sa.ns * rsub;
    if (ni < 4 && nw * 3 * slot_bytes + part <= ST_LDS_MAX) { d = 3; break; }
    if (nw * 2 * slot_bytes + part <= ST_LDS_MAX) { d = 2; break; }
    if (rsub == 1) return hipErrorNotSupported;
    --rsub;
  }
  sa.rsub = rsub;
  // x through the rings when a slice's rings hold the whole slice (fp32)
  {
    const size_t cap = (size_t)rsub * d * slot_bytes, vec = (size_t)4 * slice_cols;
    sa.xring = (a.gain && cap >= 2 * vec) ? 2 : (cap >= vec ? 1 : 0);
  }
  const int nw = sa.ns * rsub;
  const size_t lds = (size_t)nw * d * slot_bytes + part;
  switch (epi) {
    case EPI_STORE: return st_dispatch<EPI_STORE>(kf, ni, d, sa, grid, nw, lds, s);
    case EPI_RESID: return st_dispatch<EPI_RESID>(kf, ni, d, sa, grid, nw, lds, s);
    case EPI_SWIGLU: return st_dispatch<EPI_SWIGLU>(kf, ni, d, sa, grid, nw, lds, s);
    case EPI_QKV: return st_dispatch<EPI_QKV>(kf, ni, d, sa, grid, nw, lds, s);
    default: return st_dispatch<EPI_LOGITS>(kf, ni, d, sa, grid, nw, lds, s);
  }
}

hipError_t gemv_launch(int fmt_mask, int epi, const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s) {
  if (NT_GEMV_STREAM) {
    const hipError_t e = gemv_stream_launch(epi, a, n_groups, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (fmt_mask == 1 << FMT_Q4_KT || fmt_mask == 1 << FMT_Q8_0T || fmt_mask == 1 << FMT_Q5_KT) {
    int64_t weights = 0;
    for (int i = 0; i < (epi == EPI_SWIGLU ? 2 : a.nseg); ++i) weights += (int64_t)a.seg[i].rows * a.cols;
    if (weights >= 100000000) fmt_mask |= FMT_NTL;
  }
  switch (epi) {
    case EPI_STORE: return launch_mask<EPI_STORE>(fmt_mask, plan, n_groups, a, s);
    case EPI_RESID: return launch_mask<EPI_RESID>(fmt_mask, plan, n_groups, a, s);
    case EPI_SWIGLU: return launch_mask<EPI_SWIGLU>(fmt_mask, plan, n_groups, a, s);
    case EPI_QKV: return launch_mask<EPI_QKV>(fmt_mask, plan, n_groups, a, s);
    default: return launch_mask<EPI_LOGITS>(fmt_mask, plan, n_groups, a, s);
  }
}

// ---- k-token GEMM launcher
constexpr size_t GEMM_LDS_MAX = 160 * 1024 - 1024;  // dynamic LDS budget (static LDS on top)

template <int FMT, int NT>
static hipError_t gemm_launch_nt(const GemmArgs& a, hipStream_t s) {
  constexpr int NW = 16;
  auto kern = gemm_kernel<FMT, NT, NW>;
  static const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS_MAX);
  if (raised != hipSuccess) return raised;
  const size_t lds = (size_t)NT * gemm_lds_per_token(a.cols, is_float_fmt(FMT));
  constexpr int R = GEMM_ROWS<FMT, NT>;
  const int groups = (a.rows + R - 1) / R;
  const int grid = max(1, min((groups + NW - 1) / NW, num_cu()));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t gemm_launch_fmt(int nt, const GemmArgs& a, hipStream_t s) {
  if (nt <= 1) return gemm_launch_nt<FMT, 1>(a, s);
  if (nt <= 2) return gemm_launch_nt<FMT, 2>(a, s);
  if (nt <= 4) return gemm_launch_nt<FMT, 4>(a, s);
  return gemm_launch_nt<FMT, 8>(a, s);
}

#ifndef NT_GEMM_MFMA
#define NT_GEMM_MFMA 1  // Q4_K, Q5_K and Q6_K with 3 to 8 tokens on the matrix cores
#endif
static bool gemm_use_mfma(int fmt, int n_tok) {
  return NT_GEMM_MFMA && (fmt == FMT_Q4_K || fmt == FMT_Q5_K || fmt == FMT_Q6_K) && n_tok >= 3;
}

template <int FMT, int NT, int S>
static hipError_t gemm_mfma_launch_nt(const GemmArgs& a, hipStream_t s) {
  auto kern = gemm_mfma_kernel<FMT, NT, S>;
  static const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)GEMM_LDS_MAX);
  if (raised != hipSuccess) return raised;
  const int ntiles = (a.rows + 15) / 16;
  const int grid = max(1, min(ntiles, num_cu()));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(MM_NW * 64), mm_lds_bytes(FMT, NT, a.cols), s, a);
  return hipGetLastError();
}

static int gemm_mfma_chunk_cols(int fmt, int n_tok, int cols) {
  const int nt = n_tok <= 4 ? 4 : 8;
  int c = 256;  // at most 32 superblocks and NT * c <= 64 MM_NW * 64 (four staging rounds of 16 columns)
  while (c + 256 <= cols && c + 256 <= 32 * 256 && nt * (c + 256) <= 64 * MM_NW * 64 &&
         mm_lds_bytes(fmt, nt, c + 256) <= GEMM_LDS_MAX)
    c += 256;
  return c > cols ? cols : c;
}

int gemm_chunk_cols(int n_tok, int cols, int fmt) {
  const int nt = n_tok <= 1 ? 1 : n_tok <= 2 ? 2 : n_tok <= 4 ? 4 : 8;
  const bool f = is_float_fmt(fmt);
  // the widest multiple of 256 columns (a superblock, eight 32-weight blocks) whose NT
  // staged regions fit, and no wider than the matrix
  int c = 256;
  while (c + 256 <= cols && (size_t)nt * gemm_lds_per_token(c + 256, f) <= GEMM_LDS_MAX) c += 256;
  if (c > cols) c = cols;
  return c - c % col_unit(fmt);
}

hipError_t gemm_launch(int fmt, const uint8_t* w, int64_t rows, int64_t cols, int n_tok, const float* x, float* y,
                       hipStream_t s, bool accum) {
  const int be = block_elems(fmt), bb = block_bytes(fmt);
  const bool mm = gemm_use_mfma(fmt, n_tok);
  int chunk = mm ? gemm_mfma_chunk_cols(fmt, n_tok, (int)cols) : gemm_chunk_cols(n_tok, (int)cols, fmt);
  // Q4_KT chunks start at tile boundaries (16 superblocks, 4096 columns), so that each chunk's
  // tiles are laid out as those of a row of its own width
  if ((fmt == FMT_Q4_KT || fmt == FMT_Q5_KT) && chunk < cols) chunk -= chunk % 4096;
  if (fmt == FMT_Q8_0T && chunk < cols) chunk -= chunk % 2048;  // tiles of 64 blocks
  if (chunk <= 0) return hipErrorInvalidValue;
  GemmArgs a;
  a.row_bytes = (int64_t)(cols / be) * bb;
  a.rows = (int)rows;
  a.n_tok = n_tok;
  a.xld = cols;
  a.y = y;
  a.yld = rows;
  for (int64_t c0 = 0; c0 < cols; c0 += chunk) {
    a.cols = (int)(cols - c0 < chunk ? cols - c0 : chunk);
    a.w = w + (c0 / be) * bb;
    a.x = x + c0;
    a.accum = accum || c0 > 0;
    hipError_t e;
    if (mm) {
      // superblocks per wave and tile: the chunk's superblocks over the workgroup's waves
      const bool wide = a.cols > MM_NW / 2 * 256 * MM_SMAX;
      constexpr int SW = MM_SMAX, SN = MM_SMAX / 2;
      if (fmt == FMT_Q4_K)
        e = n_tok <= 4 ? (wide ? gemm_mfma_launch_nt<FMT_Q4_K, 4, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q4_K, 4, SN>(a, s))
                       : (wide ? gemm_mfma_launch_nt<FMT_Q4_K, 8, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q4_K, 8, SN>(a, s));
      else if (fmt == FMT_Q5_K)
        e = n_tok <= 4 ? (wide ? gemm_mfma_launch_nt<FMT_Q5_K, 4, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q5_K, 4, SN>(a, s))
                       : (wide ? gemm_mfma_launch_nt<FMT_Q5_K, 8, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q5_K, 8, SN>(a, s));
      else
        e = n_tok <= 4 ? (wide ? gemm_mfma_launch_nt<FMT_Q6_K, 4, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q6_K, 4, SN>(a, s))
                       : (wide ? gemm_mfma_launch_nt<FMT_Q6_K, 8, SW>(a, s) : gemm_mfma_launch_nt<FMT_Q6_K, 8, SN>(a, s));
      if (e != hipSuccess) return e;
      continue;
    }
    switch (fmt) {
      case FMT_Q8_0: e = gemm_launch_fmt<FMT_Q8_0>(n_tok, a, s); break;
      case FMT_Q4_0: e = gemm_launch_fmt<FMT_Q4_0>(n_tok, a, s); break;
      case FMT_Q4_K: e = gemm_launch_fmt<FMT_Q4_K>(n_tok, a, s); break;
      case FMT_Q4_KT: e = gemm_launch_fmt<FMT_Q4_KT>(n_tok, a, s); break;
      case FMT_Q8_0T: e = gemm_launch_fmt<FMT_Q8_0T>(n_tok, a, s); break;
      case FMT_Q5_KT: e = gemm_launch_fmt<FMT_Q5_KT>(n_tok, a, s); break;
      case FMT_Q5_K: e = gemm_launch_fmt<FMT_Q5_K>(n_tok, a, s); break;
      case FMT_F16: e = gemm_launch_fmt<FMT_F16>(n_tok, a, s); break;
      case FMT_F32: e = gemm_launch_fmt<FMT_F32>(n_tok, a, s); break;
      default: e = gemm_launch_fmt<FMT_Q6_K>(n_tok, a, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nt

