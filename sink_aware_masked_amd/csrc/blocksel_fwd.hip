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
// LDS and shared by all 64 queries x 4 heads.  Blocks go straight from memory
// into a 4-stage LDS ring (direct-to-LDS loads, two blocks at a time), stored
// line-major: row r = 8 g + rr and 16-byte chunk c = 8 L + c8 (L = which
// 128-byte half of the row) sit at byte (8 L + g) * 1024 + 128 rr +
// 16 (c8 ^ rr).  One 1-KB load instruction then fills one line of 8 rows, and
// both the 16-byte K operand reads (16 rows at one chunk) and the transposing
// V reads (8 rows x 32 bytes per half-wave) fall on distinct banks.  MFMA columns are
// (query, head) pairs: a 16-column block holds 4 queries x their 4 heads, so
// the 4 heads of a query -- which share one selection -- fill the MFMA's N
// dimension.  Per 16-column block the wave skips a staged key block unless one
// of its 4 queries selected it (wave-uniform ballot), so MFMA work follows the
// union of 4 queries' selections, not of 64.
//   S^T[key][(q,h)] = K[key][:] . Q[(q,h)][:]      (MFMA 16x16x32 bf16, Q in VGPRs)
//   O^T[dv][(q,h)] += V^T[dv][key] . P^T[key][(q,h)]
#include "common.hpp"

namespace attn {

namespace bsel {
constexpr int D = 128;
constexpr int G = 4;            // query heads per kv head
constexpr int BS = 64;          // key block size = query tile
constexpr int NW = 16;          // waves per workgroup (four per SIMD)
constexpr int NB_PER_WAVE = 1;  // 16-column blocks per wave (4 queries x 4 heads)
constexpr int NQC = D / 32;     // 4 Q^T fragments per column block
constexpr int NDV = D / 16;     // 8 output blocks
constexpr int RCH = D / 8;      // 16 16-byte chunks per row
constexpr int TILE_EL = BS * D; // bf16 elements of one K (or V) block
constexpr int LDPW = BS * RCH / 64 / NW;  // 1 direct-to-LDS load per wave per tensor
constexpr int MAXW = 32;        // selection words per query held in LDS per pass (1024 blocks)
constexpr int NSTAGE = 4;       // LDS ring: the pair of blocks computed and the pair in flight
static_assert(NSTAGE == 4, "pair r uses stages 2 (r % 2) and 2 (r % 2) + 1");
}  // namespace bsel

// 16 waves of 4 queries x 4 heads each, held to 128 registers, so four waves
// share every SIMD and one's softmax or LDS waits overlap the others' MFMAs.
template <int SINK>
__global__ __launch_bounds__(64 * bsel::NW) __attribute__((amdgpu_waves_per_eu(4, 4)))
void blocksel_fwd_bf16(const Params p) {
  using namespace bsel;
  __shared__ __attribute__((aligned(16))) bf16 kvs[NSTAGE * 2 * TILE_EL];  // stages of (K block, V block)
  __shared__ uint32_t qbits[BS][MAXW];
  __shared__ uint32_t ubits[MAXW];
  __shared__ int blist[32 * MAXW];
  __shared__ int nblist;

  // Each XCD takes a contiguous range of b (one kv head's tiles on this
  // shape).  Its tiles go last first: a tile's work grows with its position
  // in the document (the union of earlier blocks), so the long workgroups
  // start early and the short ones fill the end of the launch (2-3 %).
  const int b = xcd_remap(blockIdx.x, gridDim.x);
  const int tile = p.num_tiles - 1 - b % p.num_tiles;
  const int kvh = b / p.num_tiles;
  const int hidx = kvh / (p.Hkv / p.Hidx);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int col = lane & 15, grp = lane >> 4;
  const int q0 = tile * BS;
  const int qlast = min(q0 + BS - 1, p.T - 1);

  // candidate key blocks: from the document start of the first query to the
  // query block itself
  const SegWindow sg = seg_window(p.cu, p.num_seqs, q0, qlast);  // documents of the tile
  const int blo = sg.bound(p.cu, sg.sa) / BS;
  const int bhi = qlast / BS;
  const uint8_t* tab = p.bsel + (int64_t)hidx * p.bsel_head;

  // ---- per-lane columns: column block nb of this wave holds queries
  // q0 + 4 NB_PER_WAVE wave + 4 nb + [0, 4), lane col their (col / 4, col % 4) pair
  int qi[NB_PER_WAVE], dstart[NB_PER_WAVE];
  const int hh = col & 3;
  const int h = kvh * G + hh;
  const bf16* qg = static_cast<const bf16*>(p.q);
  const bf16* kg = static_cast<const bf16*>(p.k) + (int64_t)kvh * p.k_head;
  const bf16* vg = static_cast<const bf16*>(p.v) + (int64_t)kvh * p.v_head;
  bf16x8 qf[NB_PER_WAVE][NQC];
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    qi[nb] = q0 + 4 * NB_PER_WAVE * wave + 4 * nb + (col >> 2);
    const int qc = min(qi[nb], p.T - 1);
    dstart[nb] = 0;
    for (int s2 = sg.sa; s2 <= sg.sb; ++s2) {
      const int cs = sg.bound(p.cu, s2);
      if (qc >= cs) dstart[nb] = cs;  // last document start at or before qc
    }
    const bf16* qrow = qg + (int64_t)qc * p.q_row + (int64_t)h * p.q_head + 8 * grp;
#pragma unroll
    for (int c = 0; c < NQC; ++c) {
      qf[nb][c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);
      if (qi[nb] > qlast) qf[nb][c] = bf16x8{};
      if (p.scale_log2 < 0.0f) {  // move a negative scale into Q's sign (exact)
        typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
        qf[nb][c] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[nb][c]) ^ 0x80008000u);
      }
    }
  }

  // Per-lane LDS element offsets within a block (line-major layout above):
  // K operand rows 16*sb + col (+1024 elements per sb), chunks 4*cc + grp;
  // V^T rows 32*c2 + 4*grp + col/4 (+2048 per c2, +1024 for the second 16
  // keys), chunk pair 2n, 2n+1 of dv block n.
  const int rk = col & 7;
  int koff[NQC];
#pragma unroll
  for (int cc = 0; cc < NQC; ++cc)
    koff[cc] = ((cc >> 1) * 8 + (col >> 3)) * 512 + 64 * rk + 8 * (((4 * (cc & 1) + grp) ^ rk) & 7);
  const int rv = 4 * (grp & 1) + (col >> 2), par = (col >> 1) & 1;
  int voff[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n)
    voff[n] = (n >> 2) * 4096 + (grp >> 1) * 512 + 64 * rv + 8 * (((2 * (n & 3) + par) ^ rv) & 7) + 4 * (col & 1);

  // sl2 > 0 from here on (a negative scale sits in Q's sign; a zero scale
  // becomes the least normal float, which leaves every finite logit within
  // 2^-100 of zero, so its exp2 rounds to 1 as for the exact zero logits)
  const float sl2 = fmaxf(fabsf(p.scale_log2), __FLT_MIN__);
  const float bias2 = (SINK == kSinkKey0) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  float m2[NB_PER_WAVE], lsum[NB_PER_WAVE];
  // Kept beside the reference max m2 (updated only when it moves): thr, the
  // rescale threshold m2 + kRescaleLog2 on the raw (unscaled) logits, and
  // nmu, the exponent offset -m2 (0 while m2 is -inf)
  float thr[NB_PER_WAVE], nmu[NB_PER_WAVE];
  const float inv_sl2 = 1.0f / sl2;
  floatx4 acc[NB_PER_WAVE][NDV];
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    m2[nb] = kNegInf;
    thr[nb] = kNegInf;
    nmu[nb] = 0.0f;
    lsum[nb] = 0.0f;
#pragma unroll
    for (int n = 0; n < NDV; ++n) acc[nb][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- stage one key block (K then V, this wave's LDPW 1-KB pieces of each);
  // rows past T re-read row T-1 (finite data; masked by causality).
  // Per-lane element offsets of this wave's pieces inside a block: the
  // block's first row is a wave-uniform 64-bit base, the rest 32-bit
  // (a 64-row block spans less than 2^31 bytes).
  int kpos[LDPW], vpos[LDPW];
#pragma unroll
  for (int u = 0; u < LDPW; ++u) {
    const int i = wave * LDPW + u;  // 1-KB piece: line i >> 3 of rows 8 (i & 7) .. + 7
    const int r = 8 * (i & 7) + (lane >> 3);
    const int c = 8 * (8 * (i >> 3) + ((lane & 7) ^ (lane >> 3)));
    kpos[u] = r * (int)p.k_row + c;
    vpos[u] = r * (int)p.v_row + c;
  }
  auto issue = [&](int blk, bf16* st) {
    const uint32_t base = lds_addr(st) + (uint32_t)(wave * LDPW * 1024);
    const int64_t j0 = (int64_t)blk * BS;
    if (j0 + BS <= p.T) {  // wave-uniform: every row of the block exists
      const bf16* kb = kg + j0 * p.k_row;
      const bf16* vb = vg + j0 * p.v_row;
#pragma unroll
      for (int u = 0; u < LDPW; ++u) {
        load_lds16_m0(kb + kpos[u], base + u * 1024);
        load_lds16_m0(vb + vpos[u], base + TILE_EL * 2 + u * 1024);
      }
    } else {
#pragma unroll
      for (int u = 0; u < LDPW; ++u) {
        const int i = wave * LDPW + u;
        const int r = 8 * (i & 7) + (lane >> 3);
        const int j = min(blk * BS + r, p.T - 1);
        const int c = 8 * (8 * (i >> 3) + ((lane & 7) ^ (lane >> 3)));
        load_lds16_m0(kg + (int64_t)j * p.k_row + c, base + u * 1024);
        load_lds16_m0(vg + (int64_t)j * p.v_row + c, base + TILE_EL * 2 + u * 1024);
      }
    }
  };

  // ---- one staged block for this wave's column blocks
  auto compute = [&](int blk_, int wb, const bf16* st) {
    const int blk = __builtin_amdgcn_readfirstlane(blk_);  // wave-uniform: scalar arithmetic
    const int wsel = (blk >> 5) - wb;
    const int kb0 = blk * BS;
    const bf16* ks = st;
    const bf16* vs = st + TILE_EL;
#pragma unroll
    for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
      const int ql = 4 * NB_PER_WAVE * wave + 4 * nb + (col >> 2);
      const bool sel = (qbits[ql][wsel] >> (blk & 31)) & 1u;
      const uint64_t selm = __ballot(sel);
      if (selm == 0) continue;  // none of the 4 queries picked this block
      // Wave-uniform tests below are ballots of plain compares masked by
      // selm (scalar ands; a ballot of a compound condition costs two VALU
      // instructions more).  Is the whole block causal and inside the
      // document for every selected column?
      const bool edge = ((__ballot(kb0 < dstart[nb]) | __ballot(kb0 + BS - 1 > qi[nb])) & selm) != 0;
      const bool has_key0 =
          SINK == kSinkKey0 && (__ballot((dstart[nb] >= kb0) & (dstart[nb] < kb0 + BS)) & selm) != 0;

      // s keeps the raw dot products (unselected / masked ones -inf); the
      // scale, the key-0 bias and the reference max go into one fma in the
      // exponent, so a zero bias gives bit for bit the no-sink numbers
      float s[4][4];
      // The 16 K operands of the unit (4 key sub-blocks x 4 head-dim
      // chunks), read KP MFMAs ahead of their use.  The empty asm with a
      // memory clobber after each read keeps the scheduler from sinking the
      // reads back next to their MFMAs, which at this register budget it
      // otherwise does (one or two reads in flight).
      constexpr int KP = 3;
      auto kld = [&](int k) { return *reinterpret_cast<const bf16x8*>(ks + (k >> 2) * 1024 + koff[k & 3]); };
      bf16x8 kb[KP];
#pragma unroll
      for (int k = 0; k < KP; ++k) kb[k] = kld(k);
      floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        a = mfma32(kb[k % KP], qf[nb][k & 3], (k & 3) ? a : floatx4{0.f, 0.f, 0.f, 0.f});
        if (k + KP < 16) kb[k % KP] = kld(k + KP);
        asm volatile("" ::: "memory");
        if ((k & 3) == 3) {
#pragma unroll
          for (int e = 0; e < 4; ++e) s[k >> 2][e] = a[e];
        }
      }
      // Elementwise masks only where some selected column sees causality or a
      // document start (or the key-0 bias); otherwise a column's selection
      // acts on the whole lane: the max below ignores it and the exponent
      // takes scale 0 and offset -inf, which gives 0 for every finite logit.
      if (edge) {  // wave-uniform
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = kb0 + 16 * sb + 4 * grp + e;
            s[sb][e] = (sel & (j <= qi[nb]) & (j >= dstart[nb])) ? s[sb][e] : kNegInf;
          }
      } else if (has_key0) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[sb][e] = sel ? s[sb][e] : kNegInf;
      }
      const int dk = dstart[nb] - kb0 - 4 * grp;  // key-0 column of this lane, as 16 sb + e
      float mt = kNegInf;
      bool need;  // some column's max passed its threshold (wave-uniform)
      if (has_key0) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            mt = fmaxf(mt, __builtin_fmaf(s[sb][e], sl2, (16 * sb + e == dk) ? bias2 : 0.0f));
        need = __ballot(mt > m2[nb] + kRescaleLog2) != 0;
      } else {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
        // raw logits against the raw threshold (sl2 > 0; where rounding
        // makes the two forms disagree only the timing of a rescale moves)
        need = (__ballot(mt > thr[nb]) & selm) != 0;
      }
      // lazy rescale: a column's max passes the threshold iff one of its four
      // lanes' partial maxima does, so the lanes' exchange is only needed here
      if (need) {
        if (!has_key0) mt = sel ? mt * sl2 : kNegInf;
        const float mn = fmaxf(m2[nb], max_over_groups(mt));
        const float alpha = (m2[nb] == mn) ? 1.0f : exp2f_fast(m2[nb] - mn);
        lsum[nb] *= alpha;
#pragma unroll
        for (int n = 0; n < NDV; ++n) acc[nb][n] *= alpha;
        m2[nb] = mn;
        thr[nb] = (mn + kRescaleLog2) * inv_sl2;
        nmu[nb] = (mn == kNegInf) ? 0.0f : -mn;
      }
      float ps;
      if (has_key0) {
        const float bmu = bias2 + nmu[nb];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[sb][e] = exp2f_fast(__builtin_fmaf(s[sb][e], sl2, (16 * sb + e == dk) ? bmu : nmu[nb]));
            ps = (sb | e) ? ps + s[sb][e] : s[sb][e];
          }
      } else {
        // masked elements are already -inf (scale sl2 keeps them so); on
        // unmasked blocks an unselected column takes scale 0 and offset -inf
        const float ks = (edge | sel) ? sl2 : 0.0f, ko = (edge | sel) ? nmu[nb] : kNegInf;
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[sb][e] = exp2f_fast(__builtin_fmaf(s[sb][e], ks, ko));
            ps = (sb | e) ? ps + s[sb][e] : s[sb][e];
          }
      }
      lsum[nb] += ps;
      // P of the two 32-key halves, then the 16 P.V MFMAs as one sequence
      // with the V^T operands VP MFMAs ahead of their use, pinned as the K
      // reads are: left to itself the compiler reads each operand right
      // before its MFMA and waits for it there, so every MFMA paid a full
      // LDS round trip.
      bf16x8 pbh[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pbh[c2][e] = static_cast<bf16>(s[2 * c2][e]);
          pbh[c2][4 + e] = static_cast<bf16>(s[2 * c2 + 1][e]);
        }
      auto vld = [&](int k) {
        const bf16* v0 = vs + (k >> 3) * 2048 + voff[k & 7];
        return cat8(lds_read_tr4(v0), lds_read_tr4(v0 + 1024));
      };
      constexpr int VP = 2;  // V^T operands VP MFMAs ahead
      bf16x8 vb[VP];
#pragma unroll
      for (int k = 0; k < VP; ++k) vb[k] = vld(k);
#pragma unroll
      for (int k = 0; k < 2 * NDV; ++k) {
        const bf16x8 va = vb[k % VP];
        if (k + VP < 2 * NDV) vb[k % VP] = vld(k + VP);
        acc[nb][k & 7] = mfma32(va, pbh[k >> 3], acc[nb][k & 7]);
        asm volatile("" ::: "memory");
      }
    }
  };

  // Passes over windows of 32*MAXW candidate blocks (one window covers
  // documents up to 32*MAXW*64 tokens before the query block).
  for (int wb = blo >> 5; wb <= (bhi >> 5); wb += MAXW) {
    const int nwords = min(MAXW, (bhi >> 5) - wb + 1);
    // ---- selection bits of the 64 queries: a wave reads 64 consecutive
    // table bytes of one query row per load (one cache line, coalesced), and
    // the ballot of "byte != 0" is that row's bits for 64 blocks -- two words.
    // Eight rows' loads are issued before their ballots.
    __syncthreads();  // the previous pass is done with qbits / blist / the ring
    {
      const int nch = (nwords + 1) >> 1;  // 64-block chunks per row in this pass
      const int items = BS * nch;
      for (int it0 = wave; it0 < items; it0 += 8 * NW) {
        uint8_t v[8];
        int blk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int it = it0 + u * NW;
          const int q = it / nch, ch = it - q * nch;
          blk[u] = 32 * wb + 64 * ch + lane;
          const int qrow_idx = q0 + q;
          v[u] = 0;
          if (it < items && qrow_idx <= qlast)
            v[u] = tab[(int64_t)qrow_idx * p.bsel_q + min(max(blk[u], blo), bhi)];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int it = it0 + u * NW;
          const bool bit = (v[u] != 0) & (blk[u] >= blo) & (blk[u] <= bhi);
          const uint64_t m = __ballot(bit);
          if (it < items && lane < 2) {
            const int q = it / nch, w = 2 * (it - q * nch) + lane;
            if (w < nwords) qbits[q][w] = lane ? (uint32_t)(m >> 32) : (uint32_t)m;
          }
        }
      }
    }
    __syncthreads();
    // union over the 64 queries (a wave per word, OR-reduced across lanes),
    // then the list of blocks to stage (one wave: prefix sum of the words'
    // popcounts, each lane writing its word's blocks)
    for (int w = wave; w < nwords; w += NW) {
      uint32_t u = qbits[lane][w];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) u |= (uint32_t)__shfl_xor((int)u, off);
      if (lane == 0) ubits[w] = u;
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t bits = lane < nwords ? ubits[lane] : 0u;
      const int cnt = __builtin_popcount(bits);
      int x = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      int n = x - cnt;
      uint32_t pending = bits;
      while (pending) {
        blist[n++] = 32 * (wb + lane) + __builtin_ctz(pending);
        pending &= pending - 1;
      }
      if (lane == 63) nblist = x;
    }
    __syncthreads();
    const int nbl = nblist;

    // Blocks go in pairs: pair r lives in stages 2 (r % 2) and + 1.  One
    // wait and one barrier per pair: pair r has landed for every wave, and
    // every wave is done with pair r - 1, whose stages then take pair r + 1
    // while pair r is computed.  Between barriers a wave runs through both
    // blocks, so a wave whose queries chose neither block of a pair costs the
    // others one barrier instead of two.  Every wave issues its share of
    // the next pair after its first block of the current one: each pair
    // starts straight into compute, and the loads reach the memory pipeline
    // spread over the pair as the waves finish their first blocks (3-4 %
    // faster than issuing right after the barrier in half of the waves or in
    // all of them).
    const int npair = (nbl + 1) >> 1;
    auto issue_pair = [&](int r) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (2 * r + u < nbl) issue(blist[2 * r + u], kvs + ((r & 1) * 2 + u) * 2 * TILE_EL);
    };
    issue_pair(0);
    for (int r = 0; r < npair; ++r) {
      wait_vmcnt<0>();
      lds_barrier();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (2 * r + u < nbl) {
          compute(blist[2 * r + u], wb, kvs + ((r & 1) * 2 + u) * 2 * TILE_EL);
        }
        if (u == 0 && r + 1 < npair) issue_pair(r + 1);
      }
    }
  }

  // ---- epilogue.  Each (query, head) output row is 256 contiguous bytes;
  // the accumulators hold 4-element pieces of 16 such rows, so each wave
  // stages its 8 queries x 4 heads in the (idle) ring, rows padded by 8
  // elements, and stores them back 16 bytes per lane, whole lines.
  const float sink2 = (SINK == kSinkNull) ? __ldg(p.sinks + h) * kLog2e : 0.0f;
  constexpr int OS = D + 8;
  constexpr int ROWS = 4 * NB_PER_WAVE * G;  // (query, head) rows per wave
  static_assert(NW * ROWS * OS <= NSTAGE * 2 * TILE_EL, "staging fits the ring");
  lds_barrier();  // every wave is done with the ring
  bf16* ost = kvs + wave * ROWS * OS;
#pragma unroll
  for (int nb = 0; nb < NB_PER_WAVE; ++nb) {
    const float l = sum_over_groups(lsum[nb]);
    const float f = sink_fold<SINK>(m2[nb], l, sink2);
    const int r = 4 * (4 * nb + (col >> 2)) + hh;  // row (query, head) of this lane
#pragma unroll
    for (int n = 0; n < NDV; ++n) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = static_cast<bf16>(acc[nb][n][e] * f);
      *reinterpret_cast<bf16x4*>(ost + r * OS + 16 * n + 4 * grp) = o;
    }
    if (grp == 0 && qi[nb] <= qlast) p.lse[(int64_t)h * p.T + qi[nb]] = lse_natural(m2[nb], l);
  }
  const int qw0 = q0 + 4 * NB_PER_WAVE * wave;
#pragma unroll
  for (int u = 0; u < ROWS * RCH / 64; ++u) {
    const int c = lane + 64 * u;
    const int r = c / RCH, cc = c - r * RCH;
    const int qq = qw0 + (r >> 2), hd = kvh * G + (r & 3);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(ost + r * OS + 8 * cc);
    if (qq <= qlast)
      *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + (int64_t)qq * p.o_row + (int64_t)hd * p.o_head + 8 * cc) = v;
  }
}

int64_t blocksel_bf16_items(const Params& p) {
  return ((int64_t)p.T + bsel::BS - 1) / bsel::BS * p.Hkv * 64 * bsel::NW;
}

hipError_t launch_blocksel_bf16(const Params& p, int sink, hipStream_t st) {
  using namespace bsel;
  if (p.Dqk != D || p.Dv != D || p.group != G || p.block_size != BS || p.Hkv % p.Hidx != 0)
    return hipErrorInvalidValue;
  Params q = p;
  q.num_tiles = (p.T + BS - 1) / BS;
  const dim3 grid((unsigned)(q.num_tiles * p.Hkv)), block(64 * NW);
  switch (sink) {
    case kSinkNone: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkNone>), grid, block, 0, st, q); break;
    case kSinkKey0: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkKey0>), grid, block, 0, st, q); break;
    default: hipLaunchKernelGGL((blocksel_fwd_bf16<kSinkNull>), grid, block, 0, st, q); break;
  }
  return hipGetLastError();
}

}  // namespace attn
