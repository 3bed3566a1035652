// Stand-alone decode-path kernels: launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

hipError_t dequant_launch(int fmt, int64_t rows, int64_t cols, const void* blocks, float* w, hipStream_t s);
hipError_t repack_q4kt_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s);
hipError_t repack_q8t_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s);
hipError_t repack_q5kt_launch(int64_t rows, int64_t cols, const void* src, void* dst, hipStream_t s);
// h[t] = dequantized row token[t] of the table, for t < n_tok (rows of dim floats)
hipError_t embed_launch(int fmt, int64_t n_vocab, int64_t dim, const void* table, const int32_t* token, float* h,
                        unsigned long long* amax_reset, hipStream_t s, int n_tok = 1);
hipError_t rmsnorm_launch(int64_t n, const float* x, const float* g, float eps, float* y, hipStream_t s);
hipError_t rope_launch(int n_heads, int head_dim, int pos, double theta, float* qk, hipStream_t s);
hipError_t swiglu_launch(int64_t n, const float* gate, const float* up, float* out, hipStream_t s);
// out[t] = first index of the maximum of row t (n floats) of v, for t < n_rows
hipError_t argmax_launch(int64_t n, const float* v, int32_t* out, hipStream_t s, int n_rows = 1);
// tokens[i] = index packed in key[i], for i < n (n <= 64)
hipError_t token_from_key_launch(const unsigned long long* key, int32_t* token, hipStream_t s, int n = 1);
// key[i] = 0 for i < n (n <= 64)
hipError_t key_reset_launch(unsigned long long* key, int n, hipStream_t s);
hipError_t cosine_launch(int64_t n, const float* a, const float* b, float* out, hipStream_t s);
hipError_t read_probe_launch(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace nt
