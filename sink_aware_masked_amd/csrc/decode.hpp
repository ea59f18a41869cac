// Parameters of the sparse-MLA decode over an fp8 latent cache (mla_decode_fp8.hip).
#pragma once

#include "common.hpp"

namespace attn {

struct DecodeParams {
  const void* q;            // bf16 [T, Hq, 576]
  const void* k;            // fp8 e4m3 latent rows [Tk, 576] (row stride k_row bytes)
  const float* kv_scale;    // [Tk]
  const int32_t* topk_idx;  // [T, topk]
  const float* sinks;       // [Hq] or NULL
  void* out;                // bf16 [T, Hq, 512]
  float* lse;               // [Hq, T]
  float* ws_out;            // [nsplit, T, Hq, 512] partial outputs
  float* ws_lse;            // [nsplit, Hq, T] partial LSEs
  int64_t q_row, q_head, k_row, o_row, o_head, topk_row;
  int T, Tk, Hq, topk, nsplit, split_len;
  float scale_log2;
};

int decode_splits(int64_t T, int64_t Hq, int64_t topk);
int decode_split_len(int64_t topk, int nsplit);
hipError_t launch_mla_decode_fp8(const DecodeParams& p, int sink, hipStream_t st);

}  // namespace attn
