// Split-sequence GQA decode attention: launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nt {

struct AttnArgs {
  const float* q;          // [n_q][128]
  const uint16_t* k_cache; // [n_kv][max_ctx][128] fp16
  const uint16_t* v_cache;
  float* out;              // [n_q][128]
  float* part;             // [n_kv][n_split][G][130] partials (workspace)
  int n_kv;
  int n_ctx;
  int max_ctx;
  int n_split;
  int slots_per_wave;
};

int attn_slots_per_wave(int n_ctx, int n_kv);
int attn_n_split(int n_ctx, int slots_per_wave);
size_t attn_part_floats(int n_q, int max_ctx);  // partial floats for any n_ctx <= max_ctx
hipError_t attn_launch(const AttnArgs& a, int group, hipStream_t s);

}  // namespace nt
