// Device-side building blocks shared by the gfx950 attention kernels.
//
// The kernels compute the masked softmax with a per-head sink in the exp2
// domain: every logit is multiplied by scale*log2(e) once, the running max and
// the rescale factors are powers of two of differences of those values, and
// the natural-log LSE is recovered at the end as ln2 * (m + log2 l).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short shortx4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

enum SinkMode : int { kSinkNone = 0, kSinkKey0 = 1, kSinkNull = 2 };
enum MaskKind : int { kMaskWindow = 0, kMaskTopk = 1, kMaskBlocksel = 2 };

// Everything a kernel needs, passed by value.  Strides are in elements.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu;
  const float* sinks;
  const int32_t* topk_idx;
  const uint8_t* bsel;
  int64_t q_row, q_head, k_row, k_head, v_row, v_head, o_row, o_head;
  int64_t topk_row;
  int64_t bsel_head, bsel_q;  // strides of block_sel's index-head and query axes
  int T, Tk, Hq, Hkv, group;  // group = Hq / Hkv
  int Dqk, Dv;
  int num_seqs;
  int window;
  int topk;
  int Hidx, NB, block_size;
  float scale_log2;           // scale * log2(e)
  int num_tiles;              // query tiles per head (kernel specific)
};

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// j reads 4 consecutive 16-bit values at its own address; the group's 16 x 4
// values come back transposed so that output lane i, element r, is source
// lane 4*r + i/4's element i%4.  With source lane j pointing at
// row (r0 + j/4), column (c0 + 4*(j%4)) of a row-major tile, output lane i
// receives the column c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (shortx4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Range-checked buffer loads: a buffer resource covers `nbytes` from `base`;
// a load whose byte offset lies past the range returns zeros.  Tiles are
// staged with one resource per tile (base = the tile's first row), so tails
// past the last valid row come back as zeros without any per-lane select or
// clamped address, and the per-lane offsets are loop invariant.
constexpr int kBufferFlags = 0x00020000;  // dword3 of a raw (untyped) buffer resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nbytes, kBufferFlags);
}
__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Direct-to-LDS 16-byte loads (global_load_lds_dwordx4): lane l of the wave
// deposits its 16 bytes at lds + 16*l, so one wave instruction fills 1 KB of
// LDS contiguously; `lds` must be the same for the whole wave.  The data
// never passes through VGPRs, so several tiles can be in flight at once.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
// The same load, issued through inline assembly with an explicit M0 so that
// the compiler's own LDS-DMA tracking (which cannot always tell which LDS
// array an in-flight load targets, and then drains every load before any LDS
// read) stays out of the way: callers wait with wait_vmcnt before reading the
// destination.  `lds_addr` is the wave-uniform byte address in LDS.  M0 is
// written here; none of the kernels keep a value in M0 across these loads.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16_m0(const void* g, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_byte_addr), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt / lgkmcnt left at
// their maxima, i.e. not waited on).  Vector loads complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for hand-offs through LDS only: this wave's LDS accesses
// have completed (lgkmcnt(0)) and every wave has arrived.  Unlike
// __syncthreads it does not drain outstanding global loads (vmcnt), so
// direct-to-LDS loads issued for later tiles stay in flight across it; the
// loads a tile depends on are waited for explicitly with wait_vmcnt.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Lazy rescaling: the running reference max only moves when a new logit
// exceeds it by more than this (log2 units), so exp2(s - m) stays <= 2^8 and
// the accumulator rescale (a pass over every accumulator register) is skipped
// on almost every tile.  Exact in real arithmetic: any reference works as long
// as the terms stay in range, and the final normalisation uses the same one.
// Once P is rounded to bf16 for the P.V product it is not free: the largest
// key's weight is exactly 1 only if the reference is the running max, so a
// lazy reference adds that key's rounding error, which matters where a row
// has few keys (the window kernel follows the max at every increase instead).
constexpr float kRescaleLog2 = 8.0f;

// max / sum over the four 16-lane groups holding the same MFMA column.  The
// lane exchanges are VALU permutes (v_permlane16_swap pairs group 0 with 1
// and 2 with 3; v_permlane32_swap pairs lanes l and l + 32), not LDS round
// trips.  Each step combines a value with its partner's, so every lane ends
// with the same result (addition is commutative, so also bit for bit).
__device__ __forceinline__ float combine_swap16(float x, bool sum) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return sum ? a + b : fmaxf(a, b);
}
__device__ __forceinline__ float combine_swap32(float x, bool sum) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return sum ? a + b : fmaxf(a, b);
}
__device__ __forceinline__ float max_over_groups(float x) {
  return combine_swap32(combine_swap16(x, false), false);
}
__device__ __forceinline__ float sum_over_groups(float x) {
  return combine_swap32(combine_swap16(x, true), true);
}

// Segment s with cu[s] <= t < cu[s+1] (largest such s; empty segments are
// skipped).  Requires 0 <= t < cu[num_seqs] and cu[0] == 0.
__device__ __forceinline__ int find_segment(const int32_t* __restrict__ cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (__ldg(cu + mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Segment lookups with few dependent loads.  A chain of dependent global
// loads costs a full memory latency per link at kernel start, when every
// workgroup issues its first loads at once, so the lookups below keep the
// chain at one or two vector loads.
//
// Largest s in [0, num_seqs) with cu[s] <= t, for a wave-uniform t (the whole
// wave calls it): a 64-ary search, each level one vector load of 64 evenly
// spaced entries and a ballot (cu is non-decreasing, so the lanes with
// cu <= t form a prefix).  num_seqs <= 64 costs one load, <= 4096 two.
__device__ __forceinline__ int find_segment_w(const int32_t* __restrict__ cu, int num_seqs, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, n = num_seqs;  // invariant: cu[lo] <= t, answer in [lo, lo + n)
  while (n > 64) {
    const int step = (n + 63) >> 6;
    const int j = lane * step;
    const int v = j < n ? __ldg(cu + lo + j) : 0x7fffffff;
    const int k = 63 - __builtin_clzll(__ballot(v <= t));
    lo += k * step;
    n = min(step, n - k * step);
  }
  const int v = lane < n ? __ldg(cu + lo + lane) : 0x7fffffff;
  return lo + 63 - __builtin_clzll(__ballot(v <= t));
}

// The segments that rows [r0, r1] (wave-uniform) fall in: sa .. sb, with the
// boundaries cu[sa .. sa + 63] held one per lane, read back by readlane.
struct SegWindow {
  int sa, sb, v;  // v = cu[min(sa + lane, num_seqs)]
  // cu[s] for a wave-uniform s >= sa
  __device__ __forceinline__ int bound(const int32_t* __restrict__ cu, int s) const {
    const int j = s - sa;
    return j < 64 ? __builtin_amdgcn_readlane(v, j) : __ldg(cu + s);
  }
};
__device__ __forceinline__ SegWindow seg_window(const int32_t* __restrict__ cu, int num_seqs, int r0, int r1) {
  SegWindow w;
  const int lane = threadIdx.x & 63;
  w.sa = find_segment_w(cu, num_seqs, r0);
  w.v = __ldg(cu + min(w.sa + lane, num_seqs));
  const int k = 63 - __builtin_clzll(__ballot((w.sa + lane < num_seqs) & (w.v <= r1)));
  w.sb = k < 63 ? w.sa + k : find_segment_w(cu, num_seqs, r1);
  return w;
}

// Blocks are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// Renumber so that each XCD receives one contiguous range of logical blocks:
// neighbouring tiles, which read overlapping K/V rows, then share an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// The sink fold after the key loop, in the exp2 domain.  Returns the factor
// that turns the accumulator into the output; m2 / l are the running max and
// the row sum over the selected keys.  none / key0_bias: 1 / l.
// null_logit: m' = max(m, s), l' = l * 2^(m - m') + 2^(s - m'), factor
// 2^(m - m') / l'.  With s = -inf every step is exact (max(m, -inf) = m,
// 2^0 = 1, + 0) and the factor is bitwise the no-sink one.  Empty rows (l == 0)
// give 0.
template <int SINK>
__device__ __forceinline__ float sink_fold(float m2, float l, float sink_log2) {
  float alpha = 1.0f, ltot = l;
  if (SINK == kSinkNull) {
    const float mn = fmaxf(m2, sink_log2);
    alpha = exp2f_fast(m2 - mn);
    ltot = l * alpha + exp2f_fast(sink_log2 - mn);
  }
  return l > 0.0f ? alpha / ltot : 0.0f;
}

__device__ __forceinline__ float lse_natural(float m2, float l) {
  return l > 0.0f ? (m2 + __log2f(l)) * kLn2 : kNegInf;
}

}  // namespace attn
