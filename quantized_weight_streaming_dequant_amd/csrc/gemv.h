// Fused dequantize-and-GEMV: launch interface shared by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nt {

enum GemvEpi {
  EPI_STORE = 0,   // y[r] = (W x)[r]
  EPI_RESID = 1,   // y[r] = resid[r] + (W x)[r]; y2[r] (if set) = the same value
  EPI_SWIGLU = 2,  // seg0 = gate, seg1 = up: y[r] = silu(gate r) * (up r)
  EPI_QKV = 3,     // seg0 = q, seg1 = k, seg2 = v: RoPE on q and k, q -> q_out, k/v -> fp16 cache slot pos
  EPI_LOGITS = 4   // y[r] = (W x)[r] and a packed (value, index) max folded into *amax
};

struct GemvSeg {
  const uint8_t* w;   // blocks of this matrix
  int64_t row_bytes;
  int rows;
  int fmt;
  int grp0;           // index of this matrix's first row group in the launch
};

struct GemvArgs {
  const float* x;     // [cols]
  const float* gain;  // RMSNorm gain [cols] applied to x first, or null
  float eps;
  int cols;
  int nseg;
  GemvSeg seg[3];
  float* y;
  const float* resid;
  float* y2;
  float* q_out;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int pos;
  int max_ctx;
  double rope_theta;
  unsigned long long* amax;
};

struct GemvPlan {
  int rows_per_wave;
  int waves;
  size_t lds_bytes;
};

// Launch geometry for a format mix (bit f set for every format present) and shape.
// rows: the launch's matrix rows (0: unknown), for the choice of rows per work item.
GemvPlan gemv_plan(int epi, int cols, int fmt_mask, int rows = 0);
// Row groups (of rows_per_wave rows) a segment of `rows` rows makes under `plan`.
int gemv_groups(const GemvPlan& p, int rows);
// Enqueue.  fmt_mask: bit f set for every format present in the segments; n_groups: the
// launch's row groups over all segments.
hipError_t gemv_launch(int fmt_mask, int epi, const GemvPlan& plan, int n_groups, const GemvArgs& a, hipStream_t s);

// The streamed path's launch threshold in weights per launch (w < 0: unchanged); returns the
// previous value.
int64_t gemv_set_stream_min_weights(int64_t w);

// k-token GEMM: y[t][r] = sum_c W[r][c] x[t][c] for t < n_tok (1..GEMM_MAX_TOK), x [n_tok][cols],
// y [n_tok][rows], all device fp32; one launch per column chunk (the weights are read once).
constexpr int GEMM_MAX_TOK = 8;
// accum: add W X into y (the residual add of a decode layer) instead of overwriting it.
hipError_t gemm_launch(int fmt, const uint8_t* w, int64_t rows, int64_t cols, int n_tok, const float* x, float* y,
                       hipStream_t s, bool accum = false);
// Columns per launch of the vector-ALU k-token GEMM for n_tok tokens of format fmt.
int gemm_chunk_cols(int n_tok, int cols, int fmt);

}  // namespace nt
