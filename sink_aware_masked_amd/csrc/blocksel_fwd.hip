// Block-sparse causal attention over packed documents (MiniMax-M3-style;
// NeMo AutoModel "cp_sparse_attn" page): key j is valid for query i and head h
// iff block_sel[0, hidx(h), i, j / 64] != 0, j <= i and j lies in i's
// cu_seqlens document.  bf16, head dim 128, 64-token key blocks, 4 query heads
// per kv head; sinks: none / key0_bias / null_logit.
//
// One workgroup = 64 consecutive queries (one query block) x one kv head and
// its 4 query heads.  The selection rows of the 64 queries are packed into
// per-query bit masks in LDS (64-bit table offsets), and their union decides
// which key blocks are staged at all: each selected block is loaded once into
// LDS (K and V row-major, coalesced) and shared by all 64 queries x 4 heads.
// MFMA columns are (query, head) pairs: a 16-column block holds 4 queries x
// their 4 heads, so the 4 heads of a query -- which share one selection --
// fill the MFMA's N dimension.  Per 16-column block the wave skips a staged
// key block unless one of its 4 queries selected it (wave-uniform ballot), so
// MFMA work follows the union of 4 queries' selections, not of 64.
//   S^T[key][(q,h)] = K[key][:] . Q[(q,h)][:]      (MFMA 16x16x32 bf16, Q in VGPRs)
//   O^T[dv][(q,h)] += V^T[dv][key] . P^T[key][(q,h)]
#include "common.hpp"

namespace attn {

namespace bsel {
constexpr int D = 128;
constexpr int G = 4;          // query heads per kv head
constexpr int BS = 64;        // key block size = query tile
constexpr int NB_PER_WAVE = 4;  // 16-column blocks per wave (16 queries x 4 heads)
constexpr int NQC = D / 32;   // 4 Q^T fragments per column block
constexpr int NDV = D / 16;   // 8 output blocks
constexpr int KS = D + 8;     // K LDS row stride: 68 dwords
constexpr int VS = D + 16;    // V LDS row stride: 72 dwords
constexpr int MAXW = 32;      // selection words per query held in LDS per pass (1024 blocks)
}  // namespace bsel

template <int SINK>
__global__ __launch_bounds__(256) void blocksel_fwd_bf16(const Params p) {
  using namespace bsel;
  __shared__ __attribute__((aligned(16))) bf16 Ks[BS * KS];
  __shared__ __attribute__((aligned(16))) bf16 Vs[BS * VS];
  __shared__ uint32_t qbits[BS][MAXW];
  __shared__ uint32_t ubits[MAXW];
  __shared__ int blist[32 * MAXW];
  __shared__ int nblist;

  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = b % p.num_tiles;
  const int kvh = b / p.num_tiles;
  const int hidx = kvh / (p.Hkv / p.Hidx);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int col = lane & 15, grp = lane >> 4;
  const int q0 = tile * BS;
  const int qlast = min(q0 + BS - 1, p.T - 1);

  // candidate key blocks: from the document start of the first query to the
  // query block itself
  const int blo = __ldg(p.cu + find_segment(p.cu, p.num_seqs, q0)) / BS;
  const int bhi = qlast / BS;
  const uint8_t* tab = p.bsel + (int64_t)hidx * p.bsel_head;

  // ---- per-lane columns: n-block nb holds queries q0 + 16*wave + 4*nb + [0,4)
  int qi[NB_PER_WAVE], dstart[NB_PER_WAVE];
  const int hh = col & 3;
  const int h = kvh * G + hh;
  const bf16* qg = static_cast<const bf16*>(p.q);
  const bf16* kg = static_cast<const bf16*>(p.k);
  const bf16* vg = static_cast<const bf16*>(p.v);
  bf16x8 qf[NB_PER_WAVE][NQC];
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    qi[nb] = q0 + 16 * wave + 4 * nb + (col >> 2);
    const int qc = min(qi[nb], p.T - 1);
    dstart[nb] = __ldg(p.cu + find_segment(p.cu, p.num_seqs, qc));
    const bf16* qrow = qg + (int64_t)qc * p.q_row + (int64_t)h * p.q_head + 8 * grp;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      qf[nb][c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);
      if (qi[nb] > qlast) qf[nb][c] = bf16x8{};
    }
  }

  const float sl2 = p.scale_log2;
  const float bias2 = (SINK == kSinkKey0) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  float m2[NB_PER_WAVE], lsum[NB_PER_WAVE];
  floatx4 acc[NB_PER_WAVE][NDV];
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    m2[nb] = kNegInf;
    lsum[nb] = 0.0f;
#pragma unroll
    for (int n = 0; n < NDV; ++n) acc[nb][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // K/V staging: each thread owns NLD 16-byte chunks of a block's K and of
  // its V; the next selected block is prefetched into registers while the
  // current one is being used.
  constexpr int CH = D / 8;  // 16-byte chunks per row
  constexpr int NLD = BS * CH / 256;
  static_assert(BS * CH % 256 == 0, "whole chunks per thread");
  bf16x8 kr[NLD], vr[NLD];
  auto load_block = [&](int blk) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int t = tid + 256 * u;
      const int r = t / CH, c = t - r * CH;
      const int j = blk * BS + r;
      const bool ok = j < p.T;
      const int jc = ok ? j : p.T - 1;
      const bf16x8 kx = *reinterpret_cast<const bf16x8*>(kg + (int64_t)jc * p.k_row + (int64_t)kvh * p.k_head + 8 * c);
      const bf16x8 vx = *reinterpret_cast<const bf16x8*>(vg + (int64_t)jc * p.v_row + (int64_t)kvh * p.v_head + 8 * c);
      kr[u] = ok ? kx : bf16x8{};
      vr[u] = ok ? vx : bf16x8{};
    }
  };

  // Passes over windows of 32*MAXW candidate blocks (one window covers
  // documents up to 32*MAXW*64 tokens before the query block).
  for (int wb = blo >> 5; wb <= (bhi >> 5); wb += MAXW) {
    const int nwords = min(MAXW, (bhi >> 5) - wb + 1);
    // ---- selection bits of the 64 queries, 32 blocks per word; the 32 byte
    // loads of a word are independent (clamped index, masked bit)
    __syncthreads();  // the previous pass is done with qbits / blist / K / V
    for (int t = tid; t < BS * nwords; t += 256) {
      const int q = t / nwords, w = t - q * nwords;
      uint32_t bits = 0;
      const int qrow_idx = q0 + q;
      if (qrow_idx <= qlast) {
        const uint8_t* row = tab + (int64_t)qrow_idx * p.bsel_q;
        const int blk0 = 32 * (wb + w);
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int blk = blk0 + u;
          const uint8_t v = row[min(max(blk, blo), bhi)];
          bits |= (uint32_t)(v != 0 && blk >= blo && blk <= bhi) << u;
        }
      }
      qbits[q][w] = bits;
    }
    __syncthreads();
    // union over the 64 queries, then the list of blocks to stage
    if (tid < nwords) {
      uint32_t u = 0;
      for (int q = 0; q < BS; ++q) u |= qbits[q][tid];
      ubits[tid] = u;
    }
    __syncthreads();
    if (tid == 0) {
      int n = 0;
      for (int w = 0; w < nwords; ++w) {
        uint32_t pending = ubits[w];
        while (pending) {
          blist[n++] = 32 * (wb + w) + __builtin_ctz(pending);
          pending &= pending - 1;
        }
      }
      nblist = n;
    }
    __syncthreads();
    const int nbl = nblist;
    if (nbl > 0) load_block(blist[0]);
    for (int bi = 0; bi < nbl; ++bi) {
      const int blk = blist[bi];
      const int kb0 = blk * BS;
      const int wsel = (blk >> 5) - wb, bsel_bit = blk & 31;
      __syncthreads();  // the previous block has been consumed
#pragma unroll
      for (int u = 0; u < NLD; ++u) {
        const int t = tid + 256 * u;
        const int r = t / CH, c = t - r * CH;
        *reinterpret_cast<bf16x8*>(&Ks[r * KS + 8 * c]) = kr[u];
        *reinterpret_cast<bf16x8*>(&Vs[r * VS + 8 * c]) = vr[u];
      }
      __syncthreads();
      if (bi + 1 < nbl) load_block(blist[bi + 1]);

#pragma unroll
      for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
        const int ql = 16 * wave + 4 * nb + (col >> 2);
        const bool sel = (qbits[ql][wsel] >> bsel_bit) & 1u;
        if (__ballot(sel) == 0) continue;  // none of the 4 queries picked this block

        float s[4][4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
          floatx4 a = {0.f, 0.f, 0.f, 0.f};
          const bf16* krow = &Ks[(16 * sb + col) * KS + 8 * grp];
#pragma unroll
          for (int c = 0; c < NQC; ++c)
            a = mfma32(*reinterpret_cast<const bf16x8*>(krow + 32 * c), qf[nb][c], a);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = kb0 + 16 * sb + 4 * grp + e;
            float x = a[e] * sl2;
            if (SINK == kSinkKey0) x += (j == dstart[nb]) ? bias2 : 0.0f;
            s[sb][e] = (sel & (j <= qi[nb]) & (j >= dstart[nb])) ? x : kNegInf;
          }
        }
        float mt = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
        mt = max_over_groups(mt);
        const float mn = fmaxf(m2[nb], mt);
        const float mu = (mn == kNegInf) ? 0.0f : mn;
        const float alpha = exp2f_fast(m2[nb] - mu);
        float ps = 0.0f;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[sb][e] = exp2f_fast(s[sb][e] - mu);
            ps += s[sb][e];
          }
        lsum[nb] = lsum[nb] * alpha + ps;
        m2[nb] = mn;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          bf16x8 pb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[e] = static_cast<bf16>(s[2 * c2][e]);
            pb[4 + e] = static_cast<bf16>(s[2 * c2 + 1][e]);
          }
          const bf16* v0 = &Vs[(32 * c2 + 4 * grp + (col >> 2)) * VS + 4 * (col & 3)];
#pragma unroll
          for (int n = 0; n < NDV; ++n) {
            const bf16x8 va = cat8(lds_read_tr4(v0 + 16 * n), lds_read_tr4(v0 + 16 * VS + 16 * n));
            acc[nb][n] = mfma32(va, pb, c2 == 0 ? acc[nb][n] * alpha : acc[nb][n]);
          }
        }
      }
    }
  }

  const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    const float l = sum_over_groups(lsum[nb]);
    if (qi[nb] > qlast) continue;
    const float f = sink_fold<SINK>(m2[nb], l, sink2);
    bf16* orow = static_cast<bf16*>(p.out) + (int64_t)qi[nb] * p.o_row + (int64_t)h * p.o_head + 4 * grp;
#pragma unroll
    for (int n = 0; n < NDV; ++n) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[nb][n][e] * f);
      *reinterpret_cast<bf16x4*>(orow + 16 * n) = o;
    }
    if (grp == 0) p.lse[(int64_t)h * p.T + qi[nb]] = lse_natural(m2[nb], l);
  }
}

hipError_t launch_blocksel_bf16(const Params& p, int sink, hipStream_t st) {
  using namespace bsel;
  if (p.Dqk != D || p.Dv != D || p.group != G || p.block_size != BS || p.Hkv % p.Hidx != 0)
    return hipErrorInvalidValue;
  Params q = p;
  q.num_tiles = (p.T + BS - 1) / BS;
  const dim3 grid((unsigned)(q.num_tiles * p.Hkv)), block(256);
  switch (sink) {
    case kSinkNone: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkNone>), grid, block, 0, st, q); break;
    case kSinkKey0: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkKey0>), grid, block, 0, st, q); break;
    default: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkNull>), grid, block, 0, st, q); break;
  }
  return hipGetLastError();
}

}  // namespace attn
