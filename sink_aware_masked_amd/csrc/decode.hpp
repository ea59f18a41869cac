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

// Size of the static device scratch that holds the partial results of the
// allocation-free entry point: 96 MiB, enough for the 128-row x 64-head
// decode in 4 pieces (67.2 MB); larger calls are refused with ATTN_ERR_RANGE.
constexpr int64_t kDecodeScratchBytes = (int64_t)96 << 20;

int decode_splits(int64_t T, int64_t Hq, int64_t topk);
// Device address of the static scratch on the current device (looked up once
// per device, then cached).
hipError_t decode_scratch_address(void** addr);
int decode_split_len(int64_t topk, int nsplit);
hipError_t launch_mla_decode_fp8(const DecodeParams& p, int sink, hipStream_t st);

}  // namespace attn
