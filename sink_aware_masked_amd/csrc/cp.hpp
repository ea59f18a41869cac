// Parameters of the context-parallel reorder kernels (cp_reorder.hip).
#pragma once

#include "common.hpp"

namespace attn {

struct CpSlotsParams {
  int64_t* slots;
  int64_t t_local, n;  // n = t_local (one rank) or cp_size * t_local (all ranks)
  int cp_size, rank;   // rank < 0: every rank, rank-major
};

struct PermuteParams {
  const char* src;
  char* dst;
  const int64_t* index;
  int64_t src_row, dst_row;   // row strides in bytes
  int64_t src_rows, dst_rows;
  int64_t n;                  // rows moved (= index length)
  int chunks;                 // chunks per row
  int chunk_bytes;            // 16, 8 or 4
  int scatter;                // 0: dst[i] = src[index[i]]; 1: dst[index[i]] = src[i]
};

struct CpDocParams {
  const int64_t* positions;
  int64_t T;
  int32_t* doc_ids;   // may be NULL
  int32_t* cu;        // may be NULL; max_docs + 1 entries
  int32_t* num_docs;  // may be NULL
  int max_docs;
};

hipError_t launch_cp_slots(const CpSlotsParams& p, hipStream_t st);
hipError_t launch_permute_rows(const PermuteParams& p, hipStream_t st);
hipError_t launch_cp_documents(const CpDocParams& p, hipStream_t st);

}  // namespace attn
