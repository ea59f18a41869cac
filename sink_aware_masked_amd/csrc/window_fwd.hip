// Sliding-window attention over cu_seqlens-packed sequences, bf16, with the
// key0_bias / null_logit sinks folded in (MiMo window-attention page: the
// symmetric window inside each sequence and sinks[h] added to each sequence's
// first key; DeepSeek-V4 sparse-MLA page: the null-logit fold after the key
// loop).
//
// One workgroup = 4 waves of 32 consecutive packed query rows, arranged as
// 4 / G row blocks x G query heads of one kv head: G = 1 (128 rows x one
// head) unless the heads come in groups (GQA), where G = 4 (32 rows x four
// heads of one group) or 2 shares the staged key band between the heads.
// The key band of the workgroup, [lo(first row), hi(last row)], streams
// through LDS slots, 64 keys (K tile then V tile) per slot, filled by
// direct-to-LDS loads a round of slots at a time.  Q goes straight to VGPRs.
// Per wave and 32-key block:
//   S^T[key][row] = K[key][:] . Q[row][:]          (MFMA 32x32x16 bf16)
// so every lane owns one query row and 16 of the block's keys; masking is two
// integer compares against the row's window; the key-0 bias is one compare
// against the row's sequence start.  P (bf16) then feeds
//   O^T[dv][row] += V^T[dv][key] . P^T[key][row]   (MFMA 32x32x16 bf16)
// with V^T read straight from the row-major V tile by the transposing LDS
// read.  Blocks outside a wave's band are skipped (wave-uniform).
//
// LDS layout: rows of D bf16 (D/8 16-byte chunks), chunk c of row r stored at
// chunk (c + rot(r)) mod (D/8).  The K rotation makes the 16 rows read by one
// 16-lane quarter of a 16-byte MFMA operand read land in 16 different bank
// groups; the V rotation does the same for the 4 rows x 64 bytes that half a
// wave reads with one transposing read.  For D = 80 the V rows of one
// transposing read are taken two apart (keys 0,2,4,6 | 1,3,5,7 of each group
// of 8): that order is conflict-free with no rotation at all.  The key order
// inside a 32-key block is free (softmax and P.V sum over keys), so it is
// applied alike to the K rows of S^T and the V rows of P.V.
#include "common.hpp"

namespace attn {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

__device__ __forceinline__ floatx16 mfma32x32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct WinCfg {
  static constexpr int BM = 128;                 // rows of output staging (4 waves x 32)
  static constexpr int KT = 64;                  // keys per ring slot
  static constexpr int NCH = D / 8;              // 16-byte chunks per row
  static constexpr int NQK = D / 16;             // 32x32x16 MFMAs per block for S^T
  static constexpr int NB = (D + 31) / 32;       // 32-wide column blocks of O^T
  static constexpr int ROWB = NCH * 16;          // bytes per LDS row
  static constexpr int SLOT = 2 * KT * ROWB;     // K tile + V tile
  // resident workgroups per CU (one wave of each per SIMD).  Head dim 80 runs
  // three with two slots each: its band of 4 tiles then takes two rounds, but
  // a third workgroup hides more of each round's load wait than two more slots
  static constexpr int WG = D == 80 ? 3 : 2;
  static constexpr int NS = D == 64 ? 5 : D == 80 ? 2 : D == 96 ? 3 : 2;  // ring slots
  static constexpr int NPW = SLOT / 1024 / 4;    // 1 KB direct-to-LDS loads per wave per slot
  static constexpr bool ILV = (D == 80);         // keys two apart in one transposing read
  static_assert(NPW * 4 * 1024 == SLOT, "slot is a whole number of wave loads");
  static_assert(WG * NS * SLOT <= 160 * 1024, "WG workgroups' rings fit one CU's LDS");
  static_assert(BM * (D + 8) * 2 <= NS * SLOT, "output staging fits the ring");
};

// Chunk rotation of row r for K / Q tiles.  Row r starts at chunk phase
// (D/8) r mod 16 of the 256-byte bank space; the rows that share a phase
// (period P = 16 / gcd(D/8, 16)) are shifted apart by one chunk each, so 16
// consecutive rows read at the same logical chunk hit 16 distinct phases.
template <int D>
__device__ __forceinline__ int rot_k(int r) {
  constexpr int nch = D / 8;
  constexpr int g = (nch % 16 == 0) ? 16 : (nch % 8 == 0) ? 8 : (nch % 4 == 0) ? 4 : 2;
  constexpr int P = 16 / g;
  return (r / P) & (16 / P - 1);
}
template <int D>
__device__ __forceinline__ int rot_v(int r) {
  if (D == 64) return ((r >> 1) & 1) * 4;
  if (D == 128) return (r & 3) * 4;
  return 0;
}
// position (0..7) inside an aligned group of 8 keys for MFMA row m % 8
template <int D>
__device__ __forceinline__ int key_in8(int m) {
  return WinCfg<D>::ILV ? (((m & 3) << 1) | ((m >> 2) & 1)) : m;
}

template <int N>
__device__ __forceinline__ void wait_tiles(int k) {  // k later tiles may stay in flight
  if (k >= 3) wait_vmcnt<3 * N>();
  else if (k == 2) wait_vmcnt<2 * N>();
  else if (k == 1) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

__device__ __forceinline__ float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int SINK, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WinCfg<D>::WG, WinCfg<D>::WG)))
void window_fwd_bf16(const Params p) {
  using C = WinCfg<D>;
  static_assert(G == 1 || G == 2 || G == 4, "heads per workgroup");
  constexpr int BM = 32 * (4 / G);  // query rows per workgroup
  static_assert(D % 16 == 0 && D <= 128, "head dim");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::NS * C::SLOT];

  const int b = xcd_remap(blockIdx.x, gridDim.x);
  // tile-major: the heads of one row tile are neighbours, so an XCD's L2
  // holds whole K/V rows (all heads) of a few consecutive tiles
  const int nhg = p.Hq / G;
  const int tile = b / nhg;
  const int hg = b - tile * nhg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int n = lane & 31, hf = lane >> 5;                      // MFMA column (row of the wave), half
  const int h = G * hg + wave % G;       // this wave's query head
  const int kvh = (G * hg) / p.group;    // the G heads share it: group % G == 0
  const int r0 = tile * BM;
  const int rlast = min(r0 + BM - 1, p.T - 1);
  const int r0w = r0 + 32 * (wave / G);
  const bool wave_active = r0w <= rlast;

  // Q^T fragments (B operand) straight to VGPRs: lane (n, hf) holds row
  // r0w + n, dims 16 d + 8 hf + [0, 8).  Issued first: the rows do not
  // depend on the sequences, so the loads are in flight during the searches
  // below.
  const char* qg = static_cast<const char*>(p.q) + (int64_t)h * p.q_head * 2;
  const int64_t qrow = p.q_row * 2;
  bf16x8 qf[C::NQK];
  {
    const char* qr = qg + (int64_t)min(r0w + n, rlast) * qrow;
#pragma unroll
    for (int d = 0; d < C::NQK; ++d) qf[d] = *reinterpret_cast<const bf16x8*>(qr + 32 * d + 16 * hf);
  }

  // ---- windows.  Sequences touching this tile: sa .. sb (scalar loads).
  const int sa = find_segment(p.cu, p.num_seqs, r0);
  const int sb = find_segment(p.cu, p.num_seqs, rlast);
  // bounds as offsets that cannot overflow: max(start, r - W) = r - min(W, r - start)
  const int kmin = r0 - min(p.window, r0 - __ldg(p.cu + sa));
  const int kmax = rlast + min(p.window, __ldg(p.cu + sb + 1) - 1 - rlast);
  const int ri = min(r0w + n, rlast);  // this lane's row (clamped past the end)
  int start = 0, end = 1;
  for (int s = sa; s <= sb; ++s) {
    const int cs = __ldg(p.cu + s), ce = __ldg(p.cu + s + 1);
    if (ri >= cs && ri < ce) { start = cs; end = ce; }
  }
  const int lo = ri - min(p.window, ri - start);
  const int hi = ri + min(p.window, end - 1 - ri);
  // Rows, lo and hi are non-decreasing along the lanes 0..31.  Wave band
  // [wlo, whi]; interior [ilo, ihi] valid for every row of the wave; key-0
  // positions (sequence starts) of the wave lie in [k0a, k0b].
  const int wlo = __builtin_amdgcn_readlane(lo, 0), whi = __builtin_amdgcn_readlane(hi, 31);
  const int ilo = __builtin_amdgcn_readlane(lo, 31), ihi = __builtin_amdgcn_readlane(hi, 0);
  const int k0a = __builtin_amdgcn_readlane(start, 0), k0b = __builtin_amdgcn_readlane(start, 31);
  const int ntiles = (kmax - kmin + C::KT) / C::KT;

  // The kernel works with sl2 > 0: a negative scale is moved into Q's sign
  // (exact), and a zero scale becomes the least normal float, which leaves
  // every finite logit within 2^-100 of zero, so its exp2 rounds to 1 just as
  // for the exact zero logits.
  const bool neg_scale = p.scale_log2 < 0.0f;
  const float sl2 = fmaxf(fabsf(p.scale_log2), __FLT_MIN__);
  const float bias2 = (SINK == kSinkKey0) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;

  // ---- ring filling.  Direct-to-LDS load i of a slot (i = wave*NPW + u)
  // writes slot bytes [1024 i, 1024 i + 1024); lane l's 16 bytes land at
  // 1024 i + 16 l, i.e. physical chunk q = 64 i + l of the slot.
  const char* kg = static_cast<const char*>(p.k) + (int64_t)kvh * p.k_head * 2;
  const char* vg = static_cast<const char*>(p.v) + (int64_t)kvh * p.v_head * 2;
  const int64_t krow = p.k_row * 2, vrow = p.v_row * 2;
  const uint32_t sbase = lds_addr(smem);
  int trow[C::NPW], tc16[C::NPW];  // per load: row inside the tile, source chunk byte offset
#pragma unroll
  for (int u = 0; u < C::NPW; ++u) {
    const int i = wave * C::NPW + u;
    const bool isv = i >= C::NCH;
    const int q = 64 * (isv ? i - C::NCH : i) + lane;
    const int r = q / C::NCH, s = q - r * C::NCH;
    const int rot = isv ? rot_v<D>(r) : rot_k<D>(r);
    trow[u] = r;
    tc16[u] = 16 * ((s - rot + C::NCH) % C::NCH);
  }
  auto issue = [&](int t, int slot) {
    const int kt0 = kmin + C::KT * t;
#pragma unroll
    for (int u = 0; u < C::NPW; ++u) {
      const int i = wave * C::NPW + u;
      const bool isv = i >= C::NCH;
      const int row = min(kt0 + trow[u], kmax);  // rows past the band repeat its last key
      const char* g = (isv ? vg + row * vrow : kg + row * krow) + tc16[u];
      load_lds16_m0(g, sbase + slot * C::SLOT + 1024 * i);
    }
  };
  // ---- per-lane LDS read offsets (bytes, relative to a slot)
  constexpr int KSTEP = C::ILV ? 2 : 1;
  const int kr = (n & ~7) | key_in8<D>(n & 7);  // K row of MFMA row n in a 32-key block
  int kofs[C::NQK], vofs[C::NB];
#pragma unroll
  for (int d = 0; d < C::NQK; ++d) kofs[d] = kr * C::ROWB + 16 * ((2 * d + hf + rot_k<D>(kr)) % C::NCH);
  {
    const int j = lane & 15;
    const int vr = key_in8<D>(4 * hf + (j >> 2));  // V row (inside 8) of transposing-read row j/4
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      int col = 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      if (col >= D) col -= 16;  // D % 32 == 16: the upper half block duplicates (never stored)
      vofs[nb] = vr * C::ROWB + 16 * ((col / 8 + rot_v<D>(vr)) % C::NCH) + 2 * (col % 8);
    }
  }
  // key offset (inside a 32-key block) of accumulator element e: kbase_l + kc(e)
  const int kbase_l = C::ILV ? hf : 4 * hf;

  float m2 = kNegInf, lsum = 0.0f;
  floatx16 acc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[nb][e] = 0.0f;

  const bf16* lds = reinterpret_cast<const bf16*>(smem);
  auto compute = [&](int t, int slot) {
    const int kt0 = kmin + C::KT * t;
    if (!wave_active || kt0 > whi || kt0 + C::KT - 1 < wlo) return;  // wave-uniform
    const int kb = slot * C::SLOT, vb = kb + C::KT * C::ROWB;
    // Per 32-key block (all flags wave-uniform): live = overlaps the wave's
    // band; inside = inside every row's window (no mask); k0 = holds a key-0
    // column of some row.  x keeps the raw dot products (masked ones -inf);
    // the scale, the key-0 bias and the reference max all go into one fma in
    // the exponent, so a zero bias gives bit for bit the no-sink numbers.
    float x[2][16], bm[2];
    bool live[2], k0[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kb0 = kt0 + 32 * blk;
      live[blk] = kb0 <= whi && kb0 + 31 >= wlo;
      k0[blk] = SINK == kSinkKey0 && kb0 <= k0b && kb0 + 31 >= k0a;
      bm[blk] = kNegInf;
      if (!live[blk]) continue;
      floatx16 s = {};
#pragma unroll
      for (int d = 0; d < C::NQK; ++d)
        s = mfma32x32(*reinterpret_cast<const bf16x8*>(lds + (kb + 32 * blk * C::ROWB + kofs[d]) / 2), qf[d], s);
      if (kb0 >= ilo && kb0 + 31 <= ihi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[blk][e] = s[e];
      } else {
        const int vlo = lo - kb0 - kbase_l, vhi = hi - kb0 - kbase_l;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kc = 8 * (e >> 2) + KSTEP * (e & 3);
          x[blk][e] = ((kc >= vlo) & (kc <= vhi)) ? s[e] : kNegInf;
        }
      }
      float m = kNegInf;
      if (k0[blk]) {
        const int dk = start - kb0 - kbase_l;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kc = 8 * (e >> 2) + KSTEP * (e & 3);
          m = fmaxf(m, __builtin_fmaf(x[blk][e], sl2, kc == dk ? bias2 : 0.0f));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, x[blk][e]);
        m *= sl2;  // sl2 > 0: the max commutes with the scaling
      }
      bm[blk] = m;
    }

    // online softmax, exp2 domain.  The reference follows the running max at
    // every increase (no lazy threshold): the largest key so far then gets
    // P = 1 exactly, and only smaller weights carry the bf16 rounding of P.
    // With a lazy reference the dominant key of a short window row (up to
    // 129 keys here, often one key with a fifth of the weight) is rounded
    // too, which lifts the worst per-row error by about 30 %; the extra
    // rescale passes cost about 2 % of the kernel time.
    const float mt = swap_halves_max(fmaxf(bm[0], bm[1]));
    const float mn = fmaxf(m2, mt);
    const bool move = mn > m2;  // also m2 == -inf < mn
    if (__ballot(move) != 0) {
      const float alpha = move ? exp2f_fast(m2 - mn) : 1.0f;
      if (move) m2 = mn;
      lsum *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[nb][e] *= alpha;
    }
    const float mu = (m2 == kNegInf) ? 0.0f : m2;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (!live[blk]) continue;
      if (k0[blk]) {
        const int dk = start - (kt0 + 32 * blk) - kbase_l;
        const float bmu = bias2 - mu;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kc = 8 * (e >> 2) + KSTEP * (e & 3);
          x[blk][e] = exp2f_fast(__builtin_fmaf(x[blk][e], sl2, kc == dk ? bmu : -mu));
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[blk][e] = exp2f_fast(__builtin_fmaf(x[blk][e], sl2, -mu));
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) lsum += x[blk][e];

#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<bf16>(x[blk][8 * c2 + e]);
        const int rb = vb + (32 * blk + 16 * c2) * C::ROWB;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const bf16* v0 = lds + (rb + vofs[nb]) / 2;
          const bf16x8 va = cat8(lds_read_tr4(v0), lds_read_tr4(v0 + 8 * C::ROWB / 2));
          acc[nb] = mfma32x32(va, pb, acc[nb]);
        }
      }
    }
  };

  // ---- key loop, in rounds of NS tiles.  A round's tiles are all issued at
  // once; after one wait and one barrier every wave runs through its blocks
  // of the round without further synchronisation, so no wave waits at a
  // barrier for another wave's share of a tile it does not need itself.
  // (The 256-key band of a 64-key window on 128 rows is one round for
  // D = 64, two for D = 80.)
  // Tiles go through the rounds in the order 0, 2, 4, ..., 1, 3, ...: a
  // wave's 32 rows need a run of consecutive tiles, so each round then holds
  // about half of every wave's blocks rather than all of the first waves'.
  const int nhalf = (ntiles + 1) >> 1;
  auto tile_at = [&](int k) { return k < nhalf ? 2 * k : 2 * (k - nhalf) + 1; };
  bool first = true;
  for (int t0 = 0; t0 < ntiles; t0 += C::NS) {
    if (!first) lds_barrier();  // the previous round's slots are free
#pragma unroll
    for (int u = 0; u < C::NS; ++u)
      if (t0 + u < ntiles) issue(tile_at(t0 + u), u);
    wait_vmcnt<0>();
    lds_barrier();
    if (first && neg_scale) {
#pragma unroll
      for (int d = 0; d < C::NQK; ++d) {
        typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
        qf[d] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[d]) ^ 0x80008000u);
      }
    }
    first = false;
#pragma unroll
    for (int u = 0; u < C::NS; ++u)
      if (t0 + u < ntiles) compute(tile_at(t0 + u), u);
  }

  // ---- epilogue.  O^T leaves the accumulators as 4-element pieces of 32
  // different rows; written out directly those would be 16-byte fragments of
  // partial cache lines.  Each wave stages its 32 x D tile in LDS (rows
  // padded by 8 elements against bank conflicts) and stores it back row-major,
  // 16 bytes per lane, every row one contiguous run.
  lsum = swap_halves_sum(lsum);
  const float f = sink_fold<SINK>(m2, lsum, sink2);
  lds_barrier();  // every wave is done with the ring
  constexpr int OS = D + 8;
  bf16* ost = reinterpret_cast<bf16*>(smem) + wave * 32 * OS;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int dv = 32 * nb + 8 * q + 4 * hf;
      if (dv < D) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[nb][4 * q + e] * f);
        *reinterpret_cast<bf16x4*>(ost + n * OS + dv) = o;
      }
    }
  bf16* og = static_cast<bf16*>(p.out) + (int64_t)h * p.o_head;
  constexpr int NCHUNK = 32 * C::NCH;  // 16-byte pieces of the wave's tile
  static_assert(NCHUNK % 64 == 0, "whole wave stores");
#pragma unroll
  for (int u = 0; u < NCHUNK / 64; ++u) {
    const int c = lane + 64 * u;
    const int rr = c / C::NCH, cc = c - rr * C::NCH;
    const int row = r0w + rr;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(ost + rr * OS + 8 * cc);
    if (row <= rlast) *reinterpret_cast<bf16x8*>(og + (int64_t)row * p.o_row + 8 * cc) = v;
  }
  const int i = r0w + n;
  if (hf == 0 && i <= rlast) p.lse[(int64_t)h * p.T + i] = lse_natural(m2, lsum);
}

// Work items of one launch (workgroups x 256 lanes); every head dim uses
// 128-row tiles.
static int window_heads_per_wg(int group) { return group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1; }

int64_t window_bf16_items(const Params& p) {
  const int g = window_heads_per_wg(p.group), bm = 32 * (4 / g);
  return ((int64_t)p.T + bm - 1) / bm * (p.Hq / g) * 256;
}

template <int D, int G>
static hipError_t launch_window_dg(const Params& p, int sink, hipStream_t st) {
  Params q = p;
  constexpr int BM = 32 * (4 / G);
  q.num_tiles = (p.T + BM - 1) / BM;
  const dim3 grid((unsigned)(q.num_tiles * (p.Hq / G))), block(256);
  switch (sink) {
    case kSinkNone: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkNone, G>), grid, block, 0, st, q); break;
    case kSinkKey0: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkKey0, G>), grid, block, 0, st, q); break;
    default: hipLaunchKernelGGL((window_fwd_bf16<D, kSinkNull, G>), grid, block, 0, st, q); break;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_window_d(const Params& p, int sink, hipStream_t st) {
  switch (window_heads_per_wg(p.group)) {
    case 4: return launch_window_dg<D, 4>(p, sink, st);
    case 2: return launch_window_dg<D, 2>(p, sink, st);
    default: return launch_window_dg<D, 1>(p, sink, st);
  }
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
