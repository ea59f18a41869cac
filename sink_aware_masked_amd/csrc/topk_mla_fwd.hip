// Top-k sparse attention over one shared latent KV (DeepSeek-V4-style sparse
// MLA), bf16, with the null-logit sink folded in after the key loop
// ("Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA Triton kernel",
// Implementation paragraph).
//
// Layout: q [T, Hq, 576], kv [Tk, 1, 576] with v = kv[..., :512] (the latent
// part of the same rows), topk_idx [T, topk] int32 with -1 (or any value
// outside [0, Tk)) as padding anywhere in a row.
//
// One workgroup = one query row x 64 heads (4 waves x 16 heads); the row's
// index list is shared by all 64 heads, so each gathered 1152-byte KV row is
// staged once in LDS and used by every head.  The row's list is first
// compacted in LDS (a workgroup prefix sum over the valid entries), so padding
// costs one pass over the list and no key tiles.  Per 32-key tile and wave:
//   S^T[key][head] = K[key][:576] . Q[head][:576]   (18 MFMA 16x16x32 per 16 keys;
//                                                   Q of the wave's 16 heads in VGPRs)
//   O^T[dv][head] += V^T[dv][key] . P^T[key][head]  (32 MFMAs; V^T read from the
//                                                   same LDS rows by the transposing
//                                                   LDS read)
// Each lane owns one head for the whole softmax; the LSE is over the selected
// keys only; the sink joins the denominator in the epilogue.
#include "common.hpp"

namespace attn {

namespace mla {
constexpr int DQK = 576, DV = 512;
constexpr int HPW = 16, NW = 4, HPB = HPW * NW;   // heads per wave / per workgroup
constexpr int KT = 32;                           // keys per LDS tile
constexpr int KS = DQK + 8;                      // LDS row stride (elements)
constexpr int CHUNK = 2048;                      // list entries compacted per pass
constexpr int NQC = DQK / 32;                    // 18 Q^T fragments
constexpr int NDV = DV / 16;                     // 32 output blocks
constexpr int RCH = DQK / 8;                     // 72 16-byte chunks per KV row
}  // namespace mla

template <int SINK>
__global__ __launch_bounds__(256) void topk_mla_fwd_bf16(const Params p) {
  using namespace mla;
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KS];
  __shared__ int kidx[CHUNK];
  __shared__ int wsum[NW];

  const int ngroups = p.Hq / HPB;
  const int b = blockIdx.x;
  const int i = b / ngroups;
  const int hg = b - i * ngroups;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * HPB + wave * HPW + col;  // this lane's head

  const bf16* qg = static_cast<const bf16*>(p.q);
  const bf16* kg = static_cast<const bf16*>(p.k);
  bf16x8 qf[NQC];
  {
    const bf16* qrow = qg + (int64_t)i * p.q_row + (int64_t)h * p.q_head + 8 * grp;
#pragma unroll
    for (int c = 0; c < NQC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);
  }

  const float sl2 = p.scale_log2;
  float m2 = kNegInf, lsum = 0.0f;
  floatx4 acc[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* idx_row = p.topk_idx + (int64_t)i * p.topk_row;
  for (int c0 = 0; c0 < p.topk; c0 += CHUNK) {
    // ---- compact the valid entries of list[c0, c0 + CHUNK) into kidx[]
    __syncthreads();  // kidx / Ks of the previous pass are consumed
    int mine[CHUNK / 256];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < CHUNK / 256; ++u) {
      const int e = c0 + tid * (CHUNK / 256) + u;
      const int j = e < p.topk ? idx_row[e] : -1;
      const bool ok = j >= 0 && j < p.Tk;
      mine[u] = ok ? j : -1;
      cnt += ok;
    }
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int base = 0, nvalid = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      base += (w < wave) ? wsum[w] : 0;
      nvalid += wsum[w];
    }
    int pos = base + x - cnt;
#pragma unroll
    for (int u = 0; u < CHUNK / 256; ++u)
      if (mine[u] >= 0) kidx[pos++] = mine[u];
    __syncthreads();

    // ---- key tiles over the compacted list
    for (int t0 = 0; t0 < nvalid; t0 += KT) {
      for (int f = tid; f < KT * RCH; f += 256) {
        const int r = f / RCH, c = f - r * RCH;
        bf16x8 v = {};
        if (t0 + r < nvalid)
          v = *reinterpret_cast<const bf16x8*>(kg + (int64_t)kidx[t0 + r] * p.k_row + 8 * c);
        *reinterpret_cast<bf16x8*>(&Ks[r * KS + 8 * c]) = v;
      }
      __syncthreads();

      float s[2][4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
        const bf16* krow = &Ks[(16 * sb + col) * KS + 8 * grp];
#pragma unroll
        for (int c = 0; c < NQC; ++c)
          a = mfma32(*reinterpret_cast<const bf16x8*>(krow + 32 * c), qf[c], a);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[sb][e] = (t0 + 16 * sb + 4 * grp + e < nvalid) ? a[e] * sl2 : kNegInf;
      }
      float mt = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
      mt = max_over_groups(mt);
      const float mn = fmaxf(m2, mt);
      const float mu = (mn == kNegInf) ? 0.0f : mn;
      const float alpha = exp2f_fast(m2 - mu);
      float ps = 0.0f;
      bf16x8 pb;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = exp2f_fast(s[sb][e] - mu);
          ps += pe;
          pb[4 * sb + e] = static_cast<bf16>(pe);
        }
      lsum = lsum * alpha + ps;
      m2 = mn;
      const bf16* v0 = &Ks[(4 * grp + (col >> 2)) * KS + 4 * (col & 3)];
#pragma unroll
      for (int n = 0; n < NDV; ++n) {
        const bf16x8 va = cat8(lds_read_tr4(v0 + 16 * n), lds_read_tr4(v0 + 16 * KS + 16 * n));
        acc[n] = mfma32(va, pb, acc[n] * alpha);
      }
      __syncthreads();  // Ks consumed before the next tile is staged
    }
  }

  lsum = sum_over_groups(lsum);
  const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  const float fct = sink_fold<SINK>(m2, lsum, sink2);
  bf16* orow = static_cast<bf16*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head + 4 * grp;
#pragma unroll
  for (int n = 0; n < NDV; ++n) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[n][e] * fct);
    *reinterpret_cast<bf16x4*>(orow + 16 * n) = o;
  }
  if (grp == 0) p.lse[(int64_t)h * p.T + i] = lse_natural(m2, lsum);
}

hipError_t launch_topk_mla_bf16(const Params& p, int sink, hipStream_t st) {
  if (p.Dqk != mla::DQK || p.Dv != mla::DV || p.Hq % mla::HPB != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)p.T * (p.Hq / mla::HPB))), block(256);
  if (sink == kSinkNull)
    hipLaunchKernelGGL((topk_mla_fwd_bf16<kSinkNull>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((topk_mla_fwd_bf16<kSinkNone>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace attn
