// fp32 instance: every mask kind and sink mode, one wavefront per (row, head).
//
// This is the exact-arithmetic instance of the same contract (fp32 inputs,
// fp32 products, fp32 exp2-domain online softmax).  Each lane owns head-dim
// slots d = lane + 64*t of q, of the key being scored and of the output; the
// q.k dot product is a wavefront reduction; keys are visited one at a time
// in the order the mask enumerates them:
//   window   : the row's band [max(seq start, i-W), min(seq end-1, i+W)]
//              (MiMo window-attention page);
//   top-k    : the row's list, entries outside [0, Tk) skipped (-1 padding;
//              DeepSeek-V4 sparse-MLA page);
//   blocksel : the selected blocks of the row's index head, each clipped to
//              [document start, i] (token causal, same document; NeMo
//              "cp_sparse_attn" page), table offsets in 64-bit.
#include "common.hpp"

namespace attn {

constexpr int kGenMaxT = 9;  // up to 576 head-dim slots (64 lanes x 9)

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int MASK, int SINK>
__global__ __launch_bounds__(256) void generic_fwd_f32(const Params p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= (int64_t)p.T * p.Hq) return;  // wave-uniform
  const int i = (int)(pair / p.Hq);
  const int h = (int)(pair - (int64_t)i * p.Hq);
  const int kvh = h / p.group;
  const float* qg = static_cast<const float*>(p.q);
  const float* kg = static_cast<const float*>(p.k);
  const float* vg = static_cast<const float*>(p.v);

  float qv[kGenMaxT], acc[kGenMaxT];
  const float* qrow = qg + (int64_t)i * p.q_row + (int64_t)h * p.q_head;
#pragma unroll
  for (int t = 0; t < kGenMaxT; ++t) {
    const int d = lane + 64 * t;
    qv[t] = d < p.Dqk ? qrow[d] : 0.0f;
    acc[t] = 0.0f;
  }
  const float sl2 = p.scale_log2;
  const float bias2 = (SINK == kSinkKey0) ? p.sinks[h] * kLog2e : 0.0f;
  float m2 = kNegInf, l = 0.0f;
  int key0 = -1;

  auto visit = [&](int j) {
    const float* krow = kg + (int64_t)j * p.k_row + (int64_t)kvh * p.k_head;
    const float* vrow = vg + (int64_t)j * p.v_row + (int64_t)kvh * p.v_head;
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < kGenMaxT; ++t) {
      const int d = lane + 64 * t;
      if (d < p.Dqk) part = fmaf(qv[t], krow[d], part);
    }
    float x = wave_sum(part) * sl2;
    if (SINK == kSinkKey0 && j == key0) x += bias2;
    const float mn = fmaxf(m2, x);
    const float alpha = exp2f_fast(m2 - mn);
    const float pj = exp2f_fast(x - mn);
    l = l * alpha + pj;
#pragma unroll
    for (int t = 0; t < kGenMaxT; ++t) {
      const int d = lane + 64 * t;
      if (d < p.Dv) acc[t] = acc[t] * alpha + pj * vrow[d];
    }
    m2 = mn;
  };

  if (MASK == kMaskWindow) {
    const int s = find_segment(p.cu, p.num_seqs, i);
    const int start = p.cu[s], end = p.cu[s + 1];
    key0 = start;
    const int lo = i - min(p.window, i - start), hi = i + min(p.window, end - 1 - i);  // no overflow
    for (int j = lo; j <= hi; ++j) visit(j);
  } else if (MASK == kMaskTopk) {
    const int32_t* idx = p.topk_idx + (int64_t)i * p.topk_row;
    for (int t = 0; t < p.topk; ++t) {
      const int j = idx[t];
      if (j >= 0 && j < p.Tk) visit(j);
    }
  } else {
    const int s = find_segment(p.cu, p.num_seqs, i);
    const int start = p.cu[s];
    key0 = start;
    const int hidx = h / (p.Hq / p.Hidx);
    const uint8_t* row = p.bsel + (int64_t)hidx * p.bsel_head + (int64_t)i * p.bsel_q;
    for (int blk = start / p.block_size; blk <= i / p.block_size; ++blk) {
      if (!row[blk]) continue;
      const int a = max(start, blk * p.block_size);
      const int b = min(i, blk * p.block_size + p.block_size - 1);
      for (int j = a; j <= b; ++j) visit(j);
    }
  }

  const float sink2 = (SINK == kSinkNull) ? p.sinks[h] * kLog2e : 0.0f;
  const float f = sink_fold<SINK>(m2, l, sink2);
  float* orow = static_cast<float*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
  for (int t = 0; t < kGenMaxT; ++t) {
    const int d = lane + 64 * t;
    if (d < p.Dv) orow[d] = acc[t] * f;
  }
  if (lane == 0) p.lse[(int64_t)h * p.T + i] = lse_natural(m2, l);
}

int64_t generic_f32_items(const Params& p) { return ((int64_t)p.T * p.Hq + 3) / 4 * 256; }

template <int MASK>
static hipError_t launch_generic_m(const Params& p, int sink, hipStream_t st) {
  const int64_t pairs = (int64_t)p.T * p.Hq;
  const dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
  switch (sink) {
    case kSinkNone: hipLaunchKernelGGL((generic_fwd_f32<MASK, kSinkNone>), grid, block, 0, st, p); break;
    case kSinkKey0: hipLaunchKernelGGL((generic_fwd_f32<MASK, kSinkKey0>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((generic_fwd_f32<MASK, kSinkNull>), grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_generic_f32(const Params& p, int mask, int sink, hipStream_t st) {
  switch (mask) {
    case kMaskWindow: return launch_generic_m<kMaskWindow>(p, sink, st);
    case kMaskTopk: return launch_generic_m<kMaskTopk>(p, sink, st);
    default: return launch_generic_m<kMaskBlocksel>(p, sink, st);
  }
}

}  // namespace attn
