// The pieces of a decode layer for several tokens at consecutive positions that are not
// GEMMs (the verification pass of self-speculative decoding): launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

// y[t] = gain * x[t] / sqrt(mean(x[t]^2) + eps) for rows t < n_rows of n floats (x and y
// [n_rows][n], 16-byte aligned; n a multiple of 4 up to 32768); copy (nullable) also gets x[t].
hipError_t rmsnorm_rows_launch(int n_rows, int n, const float* x, const float* gain, float eps, float* y, float* copy,
                               hipStream_t s);

// For tokens t < n_tok at positions pos + t: RoPE on q [n_tok][n_q * 128] (in place) and on
// k [n_tok][n_kv * 128]; k and v [n_tok][n_kv * 128] rounded to fp16 into cache slot pos + t
// (K: [n_kv][max_ctx][128]; V in groups of 8 slots, [n_kv][max_ctx / 8][128][8]).
hipError_t rope_append_launch(int n_tok, int n_q, int n_kv, int pos, double theta, float* q, const float* k,
                              const float* v, uint16_t* k_cache, uint16_t* v_cache, int max_ctx, hipStream_t s);

}  // namespace nt
