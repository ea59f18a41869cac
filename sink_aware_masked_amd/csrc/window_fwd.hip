// Sliding-window attention over cu_seqlens-packed sequences, bf16, with the
// key0_bias / null_logit sinks folded in (MiMo window-attention page: the
// symmetric window inside each sequence and sinks[h] added to each sequence's
// first key; DeepSeek-V4 sparse-MLA page: the null-logit fold after the key
// loop).
//
// One workgroup = 64 consecutive packed query rows x one query head; 4 waves
// of 16 rows.  The key band of the tile, [lo(first row), hi(last row)], is
// staged through LDS in 64-key tiles (K and V row-major, coalesced 16-byte
// loads).  Per wave and 16-key sub-block:
//   S^T[key][row] = K[key][:] . Q[row][:]        (MFMA 16x16x32 bf16, Q in VGPRs)
// so every lane owns one query row; masking is two integer compares against
// the row's window [lo, hi]; the key-0 bias is one compare against the row's
// sequence start.  P (bf16) then feeds
//   O^T[dv][row] += V^T[dv][key] . P^T[key][row] (MFMA 16x16x32 bf16)
// where V^T comes straight from the row-major V tile through the transposing
// LDS read, so V is never transposed in memory.  Sub-blocks outside a wave's
// band are skipped (wave-uniform).
#include "common.hpp"

namespace attn {

template <int D>
struct WinCfg {
  static constexpr int BM = 64;                     // query rows per workgroup
  static constexpr int KT = 64;                     // keys per LDS tile
  static constexpr int NC32 = D / 32;               // full 32-wide head-dim chunks
  static constexpr bool TAIL16 = (D % 32) == 16;    // one 16-wide tail chunk
  static constexpr int NDV = D / 16;                // 16-wide output column blocks
  // Row strides (elements) chosen so that the 16-byte K reads of 8 consecutive
  // rows and the 4-row transposing V reads each hit distinct LDS banks.
  static constexpr int KS = D + 8;
  static constexpr int VS = (((D / 2) % 32) == 8 || ((D / 2) % 32) == 24) ? D : D + 16;
  // Waves per SIMD the register budget is held to: 4 resident workgroups per
  // CU keep 4 x 64 rows of one tile in flight for the small head dims.
  static constexpr int WAVES = D <= 96 ? 4 : 3;
};

template <int D, int SINK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WinCfg<D>::WAVES, WinCfg<D>::WAVES)))
void window_fwd_bf16(const Params p) {
  using C = WinCfg<D>;
  static_assert(D % 16 == 0 && D <= 256, "head dim");
  __shared__ __attribute__((aligned(16))) bf16 Ks[C::KT * C::KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[C::KT * C::VS];

  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = b % p.num_tiles;
  const int h = b / p.num_tiles;
  const int kvh = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int col = lane & 15, grp = lane >> 4;
  const int r0 = tile * C::BM;
  const int rlast = min(r0 + C::BM - 1, p.T - 1);
  const int i = r0 + wave * 16 + col;  // this lane's query row

  // Window of every row: [max(seq start, i - W), min(seq end - 1, i + W)].
  auto row_window = [&](int row, int& lo, int& hi, int& start) {
    const int s = find_segment(p.cu, p.num_seqs, row);
    start = __ldg(p.cu + s);
    lo = max(start, row - p.window);
    hi = min(__ldg(p.cu + s + 1) - 1, row + p.window);
  };
  int lo = 1, hi = 0, key0 = -1;
  if (i < p.T) row_window(i, lo, hi, key0);
  // lo and hi are non-decreasing in the row index, so the band of a set of
  // consecutive rows is [lo(first), hi(last)].
  int kmin, kmax, tmp;
  row_window(r0, kmin, tmp, tmp);
  row_window(rlast, tmp, kmax, tmp);
  // This wave's band [wlo, whi]; its interior [lo of the last row, hi of the
  // first row] is valid for every row of the wave, so sub-blocks inside it
  // need no per-element mask; key-0 positions of the wave lie in [k0a, k0b].
  int wlo = 0x7fffffff, whi = -1, ilo = 0x7fffffff, ihi = -1, k0a = -1, k0b = -1;
  {
    const int wr0 = r0 + wave * 16;
    if (wr0 <= rlast) {
      row_window(wr0, wlo, ihi, k0a);
      row_window(min(wr0 + 15, rlast), ilo, whi, k0b);
    }
  }

  // Q^T fragments (B operand): lane holds row i, dims 32c + 8*grp + [0, 8).
  const bf16* qg = static_cast<const bf16*>(p.q);
  const bf16* kg = static_cast<const bf16*>(p.k);
  const bf16* vg = static_cast<const bf16*>(p.v);
  bf16x8 qf[C::NC32 > 0 ? C::NC32 : 1];
  bf16x4 qt = {};
  {
    const bf16* qrow = qg + (int64_t)min(i, p.T - 1) * p.q_row + (int64_t)h * p.q_head;
#pragma unroll
    for (int c = 0; c < C::NC32; ++c) {
      qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c + 8 * grp);
      if (i >= p.T) qf[c] = bf16x8{};
    }
    if (C::TAIL16) {
      qt = *reinterpret_cast<const bf16x4*>(qrow + 32 * C::NC32 + 4 * grp);
      if (i >= p.T) qt = bf16x4{};
    }
  }

  const float sl2 = p.scale_log2;
  const float bias2 = (SINK == kSinkKey0) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  float m2 = kNegInf, lsum = 0.0f;
  floatx4 acc[C::NDV];
#pragma unroll
  for (int n = 0; n < C::NDV; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};

  // K/V staging: every thread owns NLD 16-byte chunks of each tile, fetched
  // with range-checked buffer loads (rows past the band come back as zeros).
  // The next tile's loads are issued right after the current tile is written
  // to LDS, so their latency overlaps this tile's MFMA work.
  constexpr int CH = D / 8;                          // 16-byte chunks per row
  constexpr int NLD = (C::KT * CH + 255) / 256;
  const bf16* kh = kg + (int64_t)kvh * p.k_head;
  const bf16* vh = vg + (int64_t)kvh * p.v_head;
  int koff[NLD], voff[NLD], lk[NLD], lv[NLD];  // global byte offsets, LDS element offsets
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int t = tid + 256 * u;
    const int r = t / CH, c = t - r * CH;
    koff[u] = (int)((r * p.k_row + 8 * c) * 2);
    voff[u] = (int)((r * p.v_row + 8 * c) * 2);
    lk[u] = r * C::KS + 8 * c;
    lv[u] = r * C::VS + 8 * c;
  }
  bf16x8 kr[NLD], vr[NLD];
  auto load_tile = [&](int kt0) {
    const int rows = min(C::KT, kmax - kt0 + 1);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (int64_t)kt0 * p.k_row, (int)(rows * p.k_row * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (int64_t)kt0 * p.v_row, (int)(rows * p.v_row * 2));
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      if (tid + 256 * u < C::KT * CH) {
        kr[u] = buf_load16(rk, koff[u]);
        vr[u] = buf_load16(rv, voff[u]);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      if (tid + 256 * u < C::KT * CH) {
        *reinterpret_cast<bf16x8*>(&Ks[lk[u]]) = kr[u];
        *reinterpret_cast<bf16x8*>(&Vs[lv[u]]) = vr[u];
      }
    }
  };

  load_tile(kmin);
  for (int kt0 = kmin; kt0 <= kmax; kt0 += C::KT) {
    __syncthreads();  // the previous tile has been consumed
    store_tile();
    __syncthreads();
    if (kt0 + C::KT <= kmax) load_tile(kt0 + C::KT);
    if (kt0 > whi || kt0 + C::KT - 1 < wlo) continue;  // wave-uniform

    float s[4][4];
    bool live[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const int kb0 = kt0 + 16 * sb;
      live[sb] = !(kb0 > whi || kb0 + 15 < wlo);
      if (!live[sb]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[sb][e] = kNegInf;
        continue;
      }
      floatx4 a = {0.f, 0.f, 0.f, 0.f};
      const bf16* krow = &Ks[(16 * sb + col) * C::KS];
#pragma unroll
      for (int c = 0; c < C::NC32; ++c)
        a = mfma32(*reinterpret_cast<const bf16x8*>(krow + 32 * c + 8 * grp), qf[c], a);
      if (C::TAIL16)
        a = mfma16(*reinterpret_cast<const bf16x4*>(krow + 32 * C::NC32 + 4 * grp), qt, a);
      const bool interior = kb0 >= ilo && kb0 + 15 <= ihi;          // wave-uniform
      const bool has_key0 = SINK == kSinkKey0 && kb0 <= k0b && kb0 + 15 >= k0a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = kb0 + 4 * grp + e;
        float x = a[e] * sl2;
        // bitwise (not short-circuit) logic: one select per element, no
        // divergent branches between the MFMA and the read of its result
        if (SINK == kSinkKey0) x += (has_key0 & (j == key0)) ? bias2 : 0.0f;
        s[sb][e] = (interior | ((j >= lo) & (j <= hi))) ? x : kNegInf;
      }
    }

    // online softmax (exp2 domain); every lane owns one row, 16 of its keys
    float mt = kNegInf;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
    mt = max_over_groups(mt);
    const float mn = fmaxf(m2, mt);
    const float mu = (mn == kNegInf) ? 0.0f : mn;
    const float alpha = exp2f_fast(m2 - mu);
    float ps = 0.0f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[sb][e] = exp2f_fast(s[sb][e] - mu);
        ps += s[sb][e];
      }
    lsum = lsum * alpha + ps;
    m2 = mn;
    if (__ballot(alpha != 1.0f) != 0) {  // skip the rescale when no row's max moved
#pragma unroll
      for (int n = 0; n < C::NDV; ++n) acc[n] *= alpha;
    }

#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      if (!live[2 * c2] && !live[2 * c2 + 1]) continue;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = static_cast<bf16>(s[2 * c2][e]);
        pb[4 + e] = static_cast<bf16>(s[2 * c2 + 1][e]);
      }
      const bf16* v0 = &Vs[(32 * c2 + 4 * grp + (col >> 2)) * C::VS + 4 * (col & 3)];
#pragma unroll
      for (int n = 0; n < C::NDV; ++n) {
        const bf16x8 va = cat8(lds_read_tr4(v0 + 16 * n), lds_read_tr4(v0 + 16 * C::VS + 16 * n));
        acc[n] = mfma32(va, pb, acc[n]);
      }
    }
  }

  lsum = sum_over_groups(lsum);
  if (i < p.T) {
    const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
    const float f = sink_fold<SINK>(m2, lsum, sink2);
    bf16* orow = static_cast<bf16*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head;
#pragma unroll
    for (int n = 0; n < C::NDV; ++n) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[n][e] * f);
      *reinterpret_cast<bf16x4*>(orow + 16 * n + 4 * grp) = o;
    }
    if (grp == 0) p.lse[(int64_t)h * p.T + i] = lse_natural(m2, lsum);
  }
}

template <int D>
static hipError_t launch_window_d(const Params& p, int sink, hipStream_t st) {
  Params q = p;
  q.num_tiles = (p.T + WinCfg<D>::BM - 1) / WinCfg<D>::BM;
  const dim3 grid((unsigned)(q.num_tiles * p.Hq)), block(256);
  switch (sink) {
    case kSinkNone: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkNone>), grid, block, 0, st, q); break;
    case kSinkKey0: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkKey0>), grid, block, 0, st, q); break;
    default: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkNull>), grid, block, 0, st, q); break;
  }
  return hipGetLastError();
}

hipError_t launch_window_bf16(const Params& p, int sink, hipStream_t st) {
  switch (p.Dqk) {
    case 64: return launch_window_d<64>(p, sink, st);
    case 80: return launch_window_d<80>(p, sink, st);
    case 96: return launch_window_d<96>(p, sink, st);
    case 128: return launch_window_d<128>(p, sink, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
