// Parameters of the kernels that act on (out, lse) pairs: the unfused key-0
// correction and the merge of partial results (compose.hip).
#pragma once

#include "common.hpp"

namespace attn {

struct Key0Params {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu;
  const float* sinks;
  int64_t q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head;
  int T, Hq, group, Dqk, Dv, num_seqs, window;
  float scale;
};

constexpr int kMergeMaxParts = 8;

struct MergeParams {
  const void* part_out[kMergeMaxParts];
  const float* part_lse[kMergeMaxParts];
  int64_t p_row[kMergeMaxParts], p_head[kMergeMaxParts];
  void* out;
  float* lse;
  const float* sinks;
  int64_t o_row, o_head;
  int T, Hq, Dv, nparts;
  int64_t nchunks;  // T * Hq * (Dv / elements per 16 bytes)
};

hipError_t launch_key0_correct(const Key0Params& p, bool f32, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, bool f32, bool null_sink, hipStream_t st);

}  // namespace attn
