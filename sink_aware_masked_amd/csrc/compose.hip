// Kernels that act on the (out, lse) pairs the attention kernels produce.
//
// key0_correct -- the unfused key-0 sink of the vLLM page "[Bugfix][MiMo]
//   Apply vision attention sinks in the window attention path" (its
//   closed-form correction paragraph): after a window attention WITHOUT sink,
//   biasing the logit of a sequence's first key by s only rescales that key's
//   softmax term, so with p0 = exp(l0 - lse) the weight the kernel gave key 0,
//       out' = (out + p0 (e^s - 1) v0) / (1 + p0 (e^s - 1)),
//   and (the LSE of the biased logits) lse' = lse + log1p(p0 (e^s - 1)).
//   Only the first W + 1 rows of a sequence see its key 0, so only they are
//   read and rewritten.  This is the comparator for the fused key0_bias path:
//   it recomputes l0 = scale q_i . k0 outside the attention kernel, as the page
//   does.
//
// merge -- combines partial results over disjoint key sets S_1 .. S_P of the
//   same query rows into the result over their union (the LSE-weighted merge
//   the MiMo page's LSE paragraph feeds through merge_attn_states):
//       lse = log sum_p e^{lse_p},  out = sum_p e^{lse_p - lse} out_p,
//   then folds a null-logit sink in once, after the merge, as the DeepSeek-V4
//   sparse-MLA page's Implementation paragraph folds it after the key loop:
//       out *= 1 / (1 + e^{s - lse}),  lse unchanged (selected keys only).
//   Partials with an empty key set (lse_p = -inf) carry no weight; if every
//   part is empty the row gets out = 0, lse = -inf.
//
// Both are bound by memory traffic (a few FLOPs per byte): one 16-byte chunk
// of a row per lane, coalesced along the head dimension.
#include "compose.hpp"

namespace attn {

template <typename E>
struct Vec16;  // 16 bytes of E, as floats
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ static void load(const void* p, float* x) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
  }
  __device__ static void store(void* p, const float* x) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(x[e]);
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, float* x) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  }
  __device__ static void store(void* p, const float* x) {
    *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
  }
};

// One wave per (affected row, head): grid.x = num_seqs * (W + 1) row slots,
// grid.y = ceil(Hq / 4) head groups of the 4 waves of a block.  Lane c < D/N
// holds 16-byte chunk c of q, k0, v0 and out; the dot product is reduced over
// the wave with xor shuffles.
template <typename E>
__global__ __launch_bounds__(256) void key0_correct_kernel(const Key0Params p) {
  using V = Vec16<E>;
  const int slot = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  const int per = p.window + 1;
  const int s = slot / per, off = slot - s * per;
  if (h >= p.Hq) return;
  const int start = p.cu[s], end = p.cu[s + 1];
  const int i = start + off;
  if (i >= end) return;  // the sequence is shorter than W + 1 rows
  const int kvh = h / p.group;
  const E* qr = static_cast<const E*>(p.q) + (int64_t)i * p.q_row + (int64_t)h * p.q_head;
  const E* kr = static_cast<const E*>(p.k) + (int64_t)start * p.k_row + (int64_t)kvh * p.k_head;
  float dot = 0.0f;
  for (int c = lane; c < p.Dqk / V::N; c += 64) {
    float a[V::N], b[V::N];
    V::load(qr + V::N * c, a);
    V::load(kr + V::N * c, b);
#pragma unroll
    for (int e = 0; e < V::N; ++e) dot = __builtin_fmaf(a[e], b[e], dot);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
  float* lse_p = p.lse + (int64_t)h * p.T + i;
  const float lse = *lse_p;
  const float p0 = expf(p.scale * dot - lse);
  const float c = p0 * expm1f(p.sinks[h]);  // p0 (e^s - 1)
  const float inv = 1.0f / (1.0f + c);
  const E* vr = static_cast<const E*>(p.v) + (int64_t)start * p.v_row + (int64_t)kvh * p.v_head;
  E* orow = static_cast<E*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head;
  for (int ch = lane; ch < p.Dv / V::N; ch += 64) {
    float o[V::N], v0[V::N];
    V::load(orow + V::N * ch, o);
    V::load(vr + V::N * ch, v0);
#pragma unroll
    for (int e = 0; e < V::N; ++e) o[e] = __builtin_fmaf(c, v0[e], o[e]) * inv;
    V::store(orow + V::N * ch, o);
  }
  if (lane == 0) *lse_p = lse + log1pf(c);
}

// One lane per 16-byte output chunk (grid-stride).
template <typename E, bool NULL_SINK>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  using V = Vec16<E>;
  const int cpr = p.Dv / V::N;  // chunks per (row, head)
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < p.nchunks; c += (int64_t)gridDim.x * 256) {
    const int64_t rh = c / cpr;
    const int d = (int)(c - rh * cpr);
    const int i = (int)(rh / p.Hq), h = (int)(rh - (int64_t)i * p.Hq);
    const int64_t li = (int64_t)h * p.T + i;
    float m = kNegInf;
    for (int q = 0; q < p.nparts; ++q) m = fmaxf(m, p.part_lse[q][li]);
    float acc[V::N] = {};
    float lse = kNegInf;
    if (m != kNegInf) {
      float wsum = 0.0f;
      for (int q = 0; q < p.nparts; ++q) {
        const float w = expf(p.part_lse[q][li] - m);
        wsum += w;
        float x[V::N];
        V::load(static_cast<const E*>(p.part_out[q]) + (int64_t)i * p.p_row[q] + (int64_t)h * p.p_head[q] + V::N * d, x);
#pragma unroll
        for (int e = 0; e < V::N; ++e) acc[e] = __builtin_fmaf(w, x[e], acc[e]);
      }
      lse = m + logf(wsum);
      float f = 1.0f / wsum;
      if (NULL_SINK) f = f / (1.0f + expf(p.sinks[h] - lse));  // s = -inf: divides by 1 exactly
#pragma unroll
      for (int e = 0; e < V::N; ++e) acc[e] *= f;
    }
    V::store(static_cast<E*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head + V::N * d, acc);
    if (d == 0) p.lse[li] = lse;
  }
}

hipError_t launch_key0_correct(const Key0Params& p, bool f32, hipStream_t st) {
  const dim3 grid((unsigned)(p.num_seqs * (p.window + 1)), (unsigned)((p.Hq + 3) / 4)), block(256);
  if (f32)
    hipLaunchKernelGGL(key0_correct_kernel<float>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(key0_correct_kernel<bf16>, grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, bool f32, bool null_sink, hipStream_t st) {
  // enough blocks to fill the chip several times over; the kernel strides
  const int64_t want = (p.nchunks + 255) / 256;
  const dim3 grid((unsigned)(want < 8192 ? want : 8192)), block(256);
  if (f32) {
    if (null_sink) hipLaunchKernelGGL((merge_kernel<float, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<float, false>), grid, block, 0, st, p);
  } else {
    if (null_sink) hipLaunchKernelGGL((merge_kernel<bf16, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((merge_kernel<bf16, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace attn
