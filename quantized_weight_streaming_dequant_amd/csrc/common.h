// Shared device helpers for the nt HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

enum { FMT_Q8_0 = 0, FMT_Q4_0 = 1, FMT_Q4_K = 2, FMT_Q6_K = 3 };

__host__ __device__ constexpr int block_elems(int f) { return f <= FMT_Q4_0 ? 32 : 256; }
__host__ __device__ constexpr int block_bytes(int f) {
  return f == FMT_Q8_0 ? 34 : f == FMT_Q4_0 ? 18 : f == FMT_Q4_K ? 144 : 210;
}

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Activation vector layout in LDS: 4 pad floats after every 64 columns, so that lanes
// reading consecutive 32- or 64-column runs with 128-bit reads spread over the banks.
__host__ __device__ __forceinline__ int xpad(int c) { return c + ((c >> 6) << 2); }
__host__ __device__ __forceinline__ int xpad_len(int cols) { return cols + (((cols + 63) >> 6) << 2); }

}  // namespace nt
