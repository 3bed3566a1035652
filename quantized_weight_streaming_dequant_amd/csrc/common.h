// Shared device helpers for the nt HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

// F16 and F32 are unquantized weight tensors: one weight per "block".  Q4_KT, Q8_0T and Q5_KT
// hold Q4_K's, Q8_0's and Q5_K's bytes rearranged in tiles (q4kt_*, q8t_*, q5kt_* below).
enum { FMT_Q8_0 = 0, FMT_Q4_0 = 1, FMT_Q4_K = 2, FMT_Q6_K = 3, FMT_Q5_K = 4, FMT_F16 = 5, FMT_F32 = 6, FMT_Q4_KT = 7,
       FMT_Q8_0T = 8, FMT_Q5_KT = 9 };
constexpr int FMT_COUNT = 10;

__host__ __device__ constexpr bool is_float_fmt(int f) { return f == FMT_F16 || f == FMT_F32; }
__host__ __device__ constexpr int block_elems(int f) { return (f <= FMT_Q4_0 || f == FMT_Q8_0T) ? 32 : is_float_fmt(f) ? 1 : 256; }
__host__ __device__ constexpr int block_bytes(int f) {
  return (f == FMT_Q8_0 || f == FMT_Q8_0T) ? 34 : f == FMT_Q4_0 ? 18 : (f == FMT_Q4_K || f == FMT_Q4_KT) ? 144 : (f == FMT_Q5_K || f == FMT_Q5_KT) ? 176 : f == FMT_F16 ? 2
         : f == FMT_F32 ? 4 : 210;
}
// Q4_KT: a row's Q4_K superblocks in tiles of 16 (the last tile of a row holds the m =
// nsb - 16 t left over), tile t at byte 2304 t of the row, so that each 16-byte load of a wave
// whose lanes take superblock j = lane / 4, quarter g = lane % 4 of a tile reads whole cache
// lines: the tile's m 16-byte headers (d, dmin, packed scales: bytes 0..15 of the Q4_K
// block) come first, then code bytes 32 g .. 32 g + 15 of each (j, g) in lane order, then
// code bytes 32 g + 16 .. 32 g + 31 in lane order (block bytes 16 + 32 g .. and 32 + 32 g ..).
// Byte offsets within the row of the three 16-byte parts of superblock b, quarter g:
__host__ __device__ constexpr uint32_t q4kt_tile_m(int nsb, int b) { return (uint32_t)(nsb - (b & ~15) < 16 ? nsb - (b & ~15) : 16); }
__host__ __device__ constexpr uint32_t q4kt_head(int nsb, int b) { return 144u * (uint32_t)(b & ~15) + 16u * (uint32_t)(b & 15); }
__host__ __device__ constexpr uint32_t q4kt_qa(int nsb, int b, int g) {
  return 144u * (uint32_t)(b & ~15) + 16u * q4kt_tile_m(nsb, b) + 16u * (4u * (uint32_t)(b & 15) + (uint32_t)g);
}
__host__ __device__ constexpr uint32_t q4kt_qb(int nsb, int b, int g) {
  return 144u * (uint32_t)(b & ~15) + 80u * q4kt_tile_m(nsb, b) + 16u * (4u * (uint32_t)(b & 15) + (uint32_t)g);
}

// Q5_KT: a row's Q5_K superblocks in tiles of 16 (m in the last), tile t at byte 2816 t: the m
// headers (bytes 0..15 of each block), the m first halves of the high bits (bytes 16..31), the
// m second halves (32..47), then code bytes 48 + 32 g .. of each (j, g) in lane order, then
// 64 + 32 g .. in lane order; the same lane work as Q5_K, each load reading whole lines.
__host__ __device__ constexpr uint32_t q5kt_base(int b) { return 176u * (uint32_t)(b & ~15); }
__host__ __device__ constexpr uint32_t q5kt_m(int nsb, int b) { return q4kt_tile_m(nsb, b); }
__host__ __device__ constexpr uint32_t q5kt_hd(int nsb, int b) { return q5kt_base(b) + 16u * (uint32_t)(b & 15); }
__host__ __device__ constexpr uint32_t q5kt_ha(int nsb, int b) { return q5kt_base(b) + 16u * q5kt_m(nsb, b) + 16u * (uint32_t)(b & 15); }
__host__ __device__ constexpr uint32_t q5kt_hb(int nsb, int b) { return q5kt_base(b) + 32u * q5kt_m(nsb, b) + 16u * (uint32_t)(b & 15); }
__host__ __device__ constexpr uint32_t q5kt_qa(int nsb, int b, int g) {
  return q5kt_base(b) + 48u * q5kt_m(nsb, b) + 16u * (4u * (uint32_t)(b & 15) + (uint32_t)g);
}
__host__ __device__ constexpr uint32_t q5kt_qb(int nsb, int b, int g) {
  return q5kt_base(b) + 112u * q5kt_m(nsb, b) + 16u * (4u * (uint32_t)(b & 15) + (uint32_t)g);
}

// Q8_0T: a row's Q8_0 blocks in tiles of 64 (the last tile of a row holds the m = nb - 64 t
// left over), tile t at byte 2176 t of the row, so that a wave whose lane l takes block l of a
// tile reads whole lines: the first 16 code bytes of each block in lane order (block bytes
// 2..17), then the second 16 (bytes 18..33), then the m fp16 scales (bytes 0..1).  Rows must
// be 16-byte multiples (cols a multiple of 256).
__host__ __device__ constexpr uint32_t q8t_tile_m(int nb, int b) { return (uint32_t)(nb - (b & ~63) < 64 ? nb - (b & ~63) : 64); }
__host__ __device__ constexpr uint32_t q8t_qa(int nb, int b) { return 34u * (uint32_t)(b & ~63) + 16u * (uint32_t)(b & 63); }
__host__ __device__ constexpr uint32_t q8t_qb(int nb, int b) {
  return 34u * (uint32_t)(b & ~63) + 16u * q8t_tile_m(nb, b) + 16u * (uint32_t)(b & 63);
}
__host__ __device__ constexpr uint32_t q8t_d(int nb, int b) {
  return 34u * (uint32_t)(b & ~63) + 32u * q8t_tile_m(nb, b) + 2u * (uint32_t)(b & 63);
}

// Column granularity of the kernels: a block, and at least 32 columns (one scale block of the
// staged activations; F16 and F32 rows are then 64- and 128-byte multiples); Q8_0T 256 columns
// (16-byte rows).
__host__ __device__ constexpr int col_unit(int f) { return f == FMT_Q8_0T ? 256 : block_elems(f) < 32 ? 32 : block_elems(f); }

// 4-byte-aligned 128/64-bit vector types: global_load_dwordx4/x2 only need dword alignment,
// and telling the compiler the true alignment keeps it from splitting or assuming more.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ uint32_t ld2(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// 16 bytes starting 2 bytes past a 4-byte boundary: two aligned loads, then byte realignment.
__device__ __forceinline__ u32x4 ld16_off2(const uint8_t* p) {
  const u32x4 a = ld16(p - 2);
  const uint32_t e = ld4(p + 14);
  u32x4 r;
  r.x = __builtin_amdgcn_alignbyte(a.y, a.x, 2);
  r.y = __builtin_amdgcn_alignbyte(a.z, a.y, 2);
  r.z = __builtin_amdgcn_alignbyte(a.w, a.z, 2);
  r.w = __builtin_amdgcn_alignbyte(e, a.w, 2);
  return r;
}

__device__ __forceinline__ u32x2 ld8_off2(const uint8_t* p) {
  const u32x2 a = ld8(p - 2);
  const uint32_t e = ld4(p + 6);
  u32x2 r;
  r.x = __builtin_amdgcn_alignbyte(a.y, a.x, 2);
  r.y = __builtin_amdgcn_alignbyte(e, a.y, 2);
  return r;
}

// fp16 bits (low 16 bits of v) -> fp32, exact.
__device__ __forceinline__ float h2f(uint32_t v) { return __half2float(__ushort_as_half((unsigned short)(v & 0xFFFFu))); }
__device__ __forceinline__ uint16_t f2h_rne(float v) { return __half_as_ushort(__float2half_rn(v)); }

// Hide a value from the optimiser so that byte extraction after a mask lowers to
// v_cvt_f32_ubyte{0,1,2,3} (extract + convert in one instruction).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }
// signed bytes -> fp32 (SDWA sign-extending converts)
__device__ __forceinline__ float sb0(uint32_t v) { return (float)(int8_t)(v & 0xFFu); }
__device__ __forceinline__ float sb1(uint32_t v) { return (float)(int8_t)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float sb2(uint32_t v) { return (float)(int8_t)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float sb3(uint32_t v) { return (float)(int8_t)(v >> 24); }

// Cross-lane moves inside rows of 16 lanes (DPP): quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.  After the four steps every lane of a row holds the row's
// reduction; the four row results are then read as scalars and combined.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_lane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Sum over the 64 lanes, returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}
// Maximum over the 64 lanes, returned to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}

// cos and sin of the RoPE angle of pair i of a head of head_dim values at position pos: the
// angle pos * theta^(-2i/head_dim) is formed and reduced to [-pi, pi] in fp64, then rounded.
__device__ __forceinline__ float2 rope_cs(double theta, int pos, int i, int head_dim) {
  const double f = pow(theta, -2.0 * (double)i / (double)head_dim);
  double ang = (double)pos * f;
  ang -= 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
  float sn, cs;
  sincosf((float)ang, &sn, &cs);
  return make_float2(cs, sn);
}

// Activation vector layout in LDS: 4 pad floats after every 64 columns and 4 more after
// every 512, so that lanes reading runs 64 columns apart (Q8_0, Q4_0, Q4_K slices) and
// runs 512 columns apart (Q6_K slices of alternate superblocks) with 128-bit reads
// spread over the banks.  Runs of 16 aligned columns stay contiguous.
__host__ __device__ __forceinline__ int xpad(int c) { return c + ((c >> 6) << 2) + ((c >> 9) << 2); }
__host__ __device__ __forceinline__ int xpad_len(int cols) { return xpad(cols + 511); }

}  // namespace nt
