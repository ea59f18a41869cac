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
// index list is shared by all 64 heads, so each gathered 1152-byte latent row
// is staged once in LDS and used by every head.  The row's list is first
// compacted in LDS (a workgroup prefix sum over the valid entries), so padding
// costs one pass over the list and no key tiles.  Key tiles of 32 gathered
// rows go straight from memory into a 2-stage LDS ring (direct-to-LDS loads,
// the next tile in flight behind the one being computed, waited for explicitly),
// stored line-major (below) so both operand reads are free of bank conflicts.
// Per tile and wave:
//   S^T[key][head] = K[key][:576] . Q[head][:576]   (18 MFMA 16x16x32 per 16 keys;
//                                                   Q of the wave's 16 heads in VGPRs)
//   O^T[dv][head] += V^T[dv][key] . P^T[key][head]  (32 MFMAs; V^T read from the
//                                                   same LDS rows by the transposing
//                                                   LDS read)
// Each lane owns one head for the whole softmax; the LSE is over the selected
// keys only; the sink joins the denominator in the epilogue.
//
// Long rows go first: the grid covers the rows twice, and a block of the first
// half computes its row only if the row's list looks long (at least a quarter
// of 64 evenly spaced entries valid), a block of the second half only if it
// does not.  Both halves evaluate the same test on the same entries, so each
// row is computed exactly once; a row of 64 tiles dispatched last would
// otherwise keep a few CUs busy alone at the end of the launch.  Q is read
// and the output written with non-temporal accesses: each is touched once, and
// the gathered latent rows should keep the caches.
#include "common.hpp"

namespace attn {

namespace mla {
constexpr int DQK = 576, DV = 512;
constexpr int HPW = 16, NW = 4, HPB = HPW * NW;   // heads per wave / per workgroup
constexpr int KT = 32;                           // keys per LDS tile
constexpr int RCH = DQK / 8;                     // 72 16-byte chunks per latent row
constexpr int TILE_CH = KT * RCH;                // 2304 chunks = 36 KB per tile
constexpr int TILE_EL = TILE_CH * 8;             // bf16 elements per tile
constexpr int NSTAGE = 2;                        // LDS ring depth
constexpr int LDPW = TILE_CH / 64 / NW;          // 9 direct-to-LDS loads per wave per tile
constexpr int CHUNK = 1024;                      // list entries compacted per pass
constexpr int NQC = DQK / 32;                    // 18 Q^T fragments
constexpr int NDV = DV / 16;                     // 32 output blocks
constexpr int KPIPE = 4;                         // K operand reads kept in flight
constexpr int VPIPE = 4;                         // V^T operand reads kept in flight
static_assert(TILE_CH % (64 * NW) == 0, "whole wave loads per tile");
}  // namespace mla

// Two workgroups per CU (LDS: 2 x 36 KB ring + a 4 KB index chunk; at most
// 256 registers per lane), so while one waits on its gathers or sits in its
// softmax the other keeps the matrix cores busy.
template <int SINK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void topk_mla_fwd_bf16(const Params p) {
  using namespace mla;
  // the two ring stages are one array: the output staging of the epilogue
  // spans both
  __shared__ __attribute__((aligned(16))) bf16 ring[NSTAGE * TILE_EL];
  bf16* const ks0 = ring;
  bf16* const ks1 = ring + TILE_EL;
  __shared__ int kidx[CHUNK];
  __shared__ int wsum[NW];

  const int ngroups = p.Hq / HPB;
  const int nhalf = p.T * ngroups;
  const int second = (int)blockIdx.x >= nhalf;
  const int b = (int)blockIdx.x - second * nhalf;
  const int i = b / ngroups;
  const int hg = b - i * ngroups;
  const int tid = threadIdx.x, lane = tid & 63;
  {
    int long_row = 0;
    if (p.topk > 0) {
      const int e = min((int)(((int64_t)lane * p.topk) >> 6), p.topk - 1);
      const int j = p.topk_idx[(int64_t)i * p.topk_row + e];
      long_row = __builtin_popcountll(__ballot(j >= 0 && j < p.Tk)) >= 16;
    }
    if (long_row == second) return;  // the other half computes this row
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * HPB + wave * HPW + col;  // this lane's head

  const bf16* qg = static_cast<const bf16*>(p.q);
  const bf16* kg = static_cast<const bf16*>(p.k);
  bf16x8 qf[NQC];
  {
    const bf16* qrow = qg + (int64_t)i * p.q_row + (int64_t)h * p.q_head + 8 * grp;
#pragma unroll
    for (int c = 0; c < NQC; ++c) qf[c] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(qrow + 32 * c));
  }

  // Tile layout in LDS, line-major: tile row r = 8 g + rr (g = 0..3) and
  // 16-byte chunk c = 8 L + c8 (L = 0..8, one 128-byte line of the row) sit
  // at byte (4 L + g) * 1024 + 128 rr + 16 (c8 ^ rr).  One 1-KB direct-to-LDS
  // load then fills one line of 8 rows, so each load instruction touches 8
  // whole cache lines (32 B pieces of 32 lines in a chunk-major layout cost
  // 15 % more time at issue), and wave g gathers rows 8 g .. 8 g + 7 — one
  // row per lane, one index read per tile.  The XOR puts the 8 rows of a
  // 16-byte operand read pass (and the 8 rows x 2 chunks of a transposing
  // read pass) in distinct bank groups.
  const int rrk = col & 7;  // K operand row in its group of 8
  const int kofs_e = ((col >> 3) * 1024 + 128 * rrk + 16 * ((grp ^ rrk) & 7)) / 2;        // even MFMA step
  const int kofs_o = ((col >> 3) * 1024 + 128 * rrk + 16 * (((4 + grp) ^ rrk) & 7)) / 2;  // odd MFMA step
  // (elements; + 2048 per pair of MFMA steps = one line, + 1024 per 16 keys)
  int vofs4[4];  // V^T reads, by output block n % 4; + 2048 per 4 blocks, + 1024 for keys + 16
  {
    const int rrv = 4 * (grp & 1) + (col >> 2), gv = grp >> 1, par = (col >> 1) & 1;
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
      vofs4[n4] = (gv * 1024 + 128 * rrv + 16 * (((2 * n4 + par) ^ rrv) & 7) + 8 * (col & 1)) / 2;
  }

  const float sl2 = p.scale_log2;
  float m2 = kNegInf, lsum = 0.0f;
  floatx4 acc[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* idx_row = p.topk_idx + (int64_t)i * p.topk_row;
  for (int c0 = 0; c0 < p.topk; c0 += CHUNK) {
    // ---- compact the valid entries of list[c0, c0 + CHUNK) into kidx[]
    __syncthreads();  // kidx / the LDS ring of the previous pass are consumed
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

    // ---- gather tile t into a stage: this wave's LDPW 1-KB pieces.  Rows
    // past the valid count re-read a valid row (finite data; their logits are
    // masked to -inf, so they carry zero weight).
    const int ntiles = (nvalid + KT - 1) / KT;
    auto issue = [&](int t, bf16* st) {
      // load u of wave w fills line u of rows 8 w .. 8 w + 7 (1 KB block 4 u + w)
      const int posr = t * KT + 8 * wave + (lane >> 3);
      const int j = kidx[posr < nvalid ? posr : 0];
      const bf16* g = kg + (int64_t)j * p.k_row + 8 * ((lane & 7) ^ (lane >> 3));
#pragma unroll
      for (int u = 0; u < LDPW; ++u) load_lds16_m0(g + 64 * u, lds_addr(st) + (4 * u + wave) * 1024);
    };

    // ---- one tile: S, online softmax with lazy rescale, PV
    auto compute = [&](int t, const bf16* st, bf16* nxt, bool late_issue) {
      const int t0 = t * KT;
      float s[2][4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
        const bf16* krow = st + 1024 * sb;
        bf16x8 kb[KPIPE];
#pragma unroll
        for (int cc = 0; cc < KPIPE; ++cc)
          kb[cc] = *reinterpret_cast<const bf16x8*>(krow + ((cc & 1) ? kofs_o : kofs_e) + 2048 * (cc >> 1));
#pragma unroll
        for (int cc = 0; cc < NQC; ++cc) {
          a = mfma32(kb[cc % KPIPE], qf[cc], a);
          const int nx = cc + KPIPE;
          if (nx < NQC)
            kb[cc % KPIPE] = *reinterpret_cast<const bf16x8*>(krow + ((nx & 1) ? kofs_o : kofs_e) + 2048 * (nx >> 1));
          asm volatile("" ::: "memory");  // keeps each read KPIPE MFMAs ahead of its use
        }
        const bool all_in = t0 + 16 * sb + 4 * grp + 3 < nvalid;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[sb][e] = (all_in | (t0 + 16 * sb + 4 * grp + e < nvalid)) ? a[e] * sl2 : kNegInf;
      }
      float mt = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
      // lazy rescale (wave-uniform; the lanes' maxima are exchanged only on
      // that path: a column passes the threshold iff one of its lanes does)
      if (__ballot(mt > m2 + kRescaleLog2) != 0) {
        const float mn = fmaxf(m2, max_over_groups(mt));
        const float alpha = (m2 == mn) ? 1.0f : exp2f_fast(m2 - mn);
        lsum *= alpha;
#pragma unroll
        for (int n = 0; n < NDV; ++n) acc[n] *= alpha;
        m2 = mn;
      }
      const float mu = (m2 == kNegInf) ? 0.0f : m2;
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
      lsum += ps;
      if (late_issue) issue(t + 1, nxt);  // waves 2-3: the next tile's gathers after the softmax
      // V^T operands run VPIPE blocks ahead of the MFMAs that use them
      auto vload = [&](int n) {
        const bf16* v0 = st + vofs4[n & 3] + 2048 * (n >> 2);
        return cat8(lds_read_tr4(v0), lds_read_tr4(v0 + 1024));
      };
      bf16x8 vb[VPIPE];
#pragma unroll
      for (int n = 0; n < VPIPE; ++n) vb[n] = vload(n);
#pragma unroll
      for (int n = 0; n < NDV; ++n) {
        acc[n] = mfma32(vb[n % VPIPE], pb, acc[n]);
        if (n + VPIPE < NDV) vb[n % VPIPE] = vload(n + VPIPE);
      }
    };

    // tile t lives in stage t % 2; the loop is unrolled by the ring depth so
    // every LDS access names its stage array at compile time
    // Waves 0-1 issue the next tile's gathers right after the barrier, waves
    // 2-3 after their softmax, so a tile's 36 gather instructions reach the
    // memory pipeline in two bursts (~1 % faster than one).
    const bool late = wave >= 2;  // wave-uniform
    auto step = [&](int t, bf16* cur, bf16* next) {
      wait_vmcnt<0>();
      lds_barrier();  // tile t is in LDS for every wave; tile t-1's stage is free
      const bool more = t + 1 < ntiles;
      if (more && !late) issue(t + 1, next);
      compute(t, cur, next, more && late);
    };
    if (ntiles > 0) issue(0, ks0);
    for (int t = 0; t < ntiles; t += NSTAGE) {
      step(t, ks0, ks1);
      if (t + 1 < ntiles) step(t + 1, ks1, ks0);
    }
  }

  lsum = sum_over_groups(lsum);
  const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  const float fct = sink_fold<SINK>(m2, lsum, sink2);
  if (grp == 0) p.lse[(int64_t)h * p.T + i] = lse_natural(m2, lsum);

  // The 64 heads of a row are one contiguous 64 KB run of out.  Each wave
  // stages its 16 x 512 tile in the (now idle) ring, rows padded by 8
  // elements, and writes it back 16 bytes per lane in address order, so the
  // stores are whole cache lines instead of 32-byte pieces of 16 rows.
  constexpr int OS = DV + 8;
  lds_barrier();  // every wave is done with the ring
  bf16* ost = ks0 + wave * (HPW * OS);
  static_assert(NW * HPW * OS <= NSTAGE * TILE_EL, "staging fits the ring");
#pragma unroll
  for (int n = 0; n < NDV; ++n) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[n][e] * fct);
    *reinterpret_cast<bf16x4*>(ost + col * OS + 16 * n + 4 * grp) = o;
  }
  bf16* og = static_cast<bf16*>(p.out) + (int64_t)i * p.o_row + (int64_t)(hg * HPB + wave * HPW) * p.o_head;
#pragma unroll
  for (int u = 0; u < HPW * DV / 8 / 64; ++u) {
    const int c = lane + 64 * u;              // 16-byte piece of the wave's tile
    const int hh = c / (DV / 8), cc = c - hh * (DV / 8);
    __builtin_nontemporal_store(*reinterpret_cast<const bf16x8*>(ost + hh * OS + 8 * cc),
                                reinterpret_cast<bf16x8*>(og + (int64_t)hh * p.o_head + 8 * cc));
  }
}

int64_t topk_mla_bf16_items(const Params& p) { return 2 * (int64_t)p.T * (p.Hq / mla::HPB) * 256; }

hipError_t launch_topk_mla_bf16(const Params& p, int sink, hipStream_t st) {
  if (p.Dqk != mla::DQK || p.Dv != mla::DV || p.Hq % mla::HPB != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(2 * (int64_t)p.T * (p.Hq / mla::HPB))), block(256);  // two passes, see above
  if (sink == kSinkNull)
    hipLaunchKernelGGL((topk_mla_fwd_bf16<kSinkNull>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((topk_mla_fwd_bf16<kSinkNone>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace attn
