// Split-sequence GQA decode attention: launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nt.h"

namespace nt {

// Largest cache capacity the split merge supports (its per-split maxima and sums sit in LDS).
constexpr int ATTN_MAX_CTX = NT_MAX_CTX;

struct AttnArgs {
  const float* q;          // [n_q][128]
  const uint16_t* k_cache; // [n_kv][max_ctx][128] fp16
  const uint16_t* v_cache; // [n_kv][max_ctx/8][128][8] fp16
  float* out;              // [n_q][128]
  float* part;             // [n_kv][n_split][G][130] partials per token (workspace)
  int n_kv;
  int n_ctx;
  int max_ctx;             // multiple of 8, <= ATTN_MAX_CTX
  int n_split;             // attn_n_split(n_ctx + n_tok - 1): the most splits of any token
  // Several query tokens at consecutive positions (the verification pass of self-speculative
  // decoding): token t attends over slots [0, n_ctx + t); its query, output and partials sit
  // t * q_stride, t * out_stride and t * part_stride floats on.
  int n_tok = 1;
  int64_t q_stride = 0, out_stride = 0, part_stride = 0;
};

int attn_n_split(int n_ctx);
size_t attn_part_floats(int n_q, int max_ctx);  // partial floats for any n_ctx <= max_ctx
hipError_t attn_launch(const AttnArgs& a, int group, hipStream_t s);

}  // namespace nt
