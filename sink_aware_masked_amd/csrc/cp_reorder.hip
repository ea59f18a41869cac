// Context-parallel reorder primitives of the NeMo AutoModel "cp_sparse_attn"
// API page, as device kernels, so that K/V gathered from load-balanced CP
// shards can be put into global token order (and back), and packed position
// ids turned into document ids and the cu_seqlens the attention kernels take,
// without a host round trip.
//
// cp_slots      cp_load_balanced_global_slots: the sequence is cut into
//               2 * cp_size equal chunks and rank r holds chunks r and
//               2 * cp_size - 1 - r, in that order; rank < 0 gives the slots
//               of every rank, rank-major (the all-gathered concatenation).
// permute_rows  order_by_positions (scatter: dst[index[i]] = src[i]) and
//               restore_by_positions (gather: dst[i] = src[index[i]]) on
//               whole rows of a [rows, ...] tensor, in 16-, 8- or 4-byte
//               chunks (the widest that divides the row and its alignment).
// documents     cp_document_ids = cumsum(positions == 0) - 1, and the
//               segment boundaries (token 0 and every later position-0 token,
//               then T) in one pass of a single workgroup (16 positions
//               per thread per step).
//
// All three are bound by memory traffic; permute_rows moves each row once,
// coalesced along the row.
#include "cp.hpp"

namespace attn {

__global__ __launch_bounds__(256) void cp_slots_kernel(const CpSlotsParams p) {
  const int64_t c = p.t_local / 2;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < p.n; g += (int64_t)gridDim.x * 256) {
    const int64_t r = p.rank >= 0 ? p.rank : g / p.t_local;
    const int64_t j = p.rank >= 0 ? g : g - r * p.t_local;
    p.slots[g] = j < c ? r * c + j : (2 * (int64_t)p.cp_size - 1 - r) * c + (j - c);
  }
}

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
template <int B> struct Chunk;
template <> struct Chunk<16> { typedef u32x4 T; };
template <> struct Chunk<8> { typedef u32x2 T; };
template <> struct Chunk<4> { typedef unsigned T; };

// Rows move in chunks of B bytes (16 where the row length allows, else 8 or 4).
template <int B>
__global__ __launch_bounds__(256) void permute_rows_kernel(const PermuteParams p) {
  typedef typename Chunk<B>::T C;
  const int64_t total = p.n * p.chunks;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t i = c / p.chunks;
    const int k = (int)(c - i * p.chunks);
    const int64_t j = p.index[i];
    if (p.scatter) {
      if (j < 0 || j >= p.dst_rows) continue;  // out-of-range target: row dropped
      const C v = *reinterpret_cast<const C*>(p.src + i * p.src_row + B * k);
      *reinterpret_cast<C*>(p.dst + j * p.dst_row + B * k) = v;
    } else {
      C v = {};                                  // out-of-range source: zero row
      if (j >= 0 && j < p.src_rows) v = *reinterpret_cast<const C*>(p.src + j * p.src_row + B * k);
      *reinterpret_cast<C*>(p.dst + i * p.dst_row + B * k) = v;
    }
  }
}

// One workgroup of 1024 threads walks the positions in tiles of 1024 x 16:
// each thread counts its 16 consecutive positions, a block-wide exclusive
// scan of the per-thread counts (two counts packed in one int: low 16 bits
// position-0 tokens, high 16 bits segment starts; a tile holds at most 16384
// of each) gives its starting point on top of the earlier tiles' totals, and
// the thread then writes its 16 ids and its segment starts.
__global__ __launch_bounds__(1024) void cp_documents_kernel(const CpDocParams p) {
  constexpr int ITEMS = 16, TILE = 1024 * ITEMS;
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry_z = 0, carry_s = 0;  // identical in every thread
  for (int64_t base = 0; base < p.T; base += TILE) {
    const int64_t i0 = base + (int64_t)tid * ITEMS;
    unsigned zbits = 0, sbits = 0;
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int64_t i = i0 + u;
      if (i < p.T) {
        const int64_t pos = p.positions[i];
        zbits |= (unsigned)(pos == 0) << u;
        sbits |= (unsigned)(pos == 0 || i == 0) << u;
      }
    }
    const int mine = (__builtin_popcount(sbits) << 16) | __builtin_popcount(zbits);
    int x = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, tile = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      before += (w < wave) ? wsum[w] : 0;
      tile += wsum[w];
    }
    const int excl = before + x - mine;
    int zi = carry_z + (excl & 0xffff), si = carry_s + (excl >> 16);
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int64_t i = i0 + u;
      if (i < p.T) {
        zi += (zbits >> u) & 1;
        if ((sbits >> u) & 1) {
          if (p.cu && si < p.max_docs) p.cu[si] = (int32_t)i;
          ++si;
        }
        if (p.doc_ids) p.doc_ids[i] = zi - 1;
      }
    }
    carry_z += tile & 0xffff;
    carry_s += tile >> 16;
    __syncthreads();  // wsum is rewritten by the next tile
  }
  if (tid == 0) {
    if (p.cu && carry_s <= p.max_docs) p.cu[carry_s] = (int32_t)p.T;
    if (p.num_docs) *p.num_docs = carry_s;
  }
}

static unsigned grid_for(int64_t items) {
  const int64_t b = (items + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b < 16384 ? b : 16384));
}

hipError_t launch_cp_slots(const CpSlotsParams& p, hipStream_t st) {
  hipLaunchKernelGGL(cp_slots_kernel, dim3(grid_for(p.n)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const PermuteParams& p, hipStream_t st) {
  const dim3 grid(grid_for(p.n * p.chunks)), block(256);
  switch (p.chunk_bytes) {
    case 16: hipLaunchKernelGGL(permute_rows_kernel<16>, grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL(permute_rows_kernel<8>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(permute_rows_kernel<4>, grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_cp_documents(const CpDocParams& p, hipStream_t st) {
  hipLaunchKernelGGL(cp_documents_kernel, dim3(1), dim3(1024), 0, st, p);
  return hipGetLastError();
}

}  // namespace attn
