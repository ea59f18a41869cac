// Sparse-MLA decode over an fp8 latent KV cache, with the null-logit sink
// folded in after all keys ("Apply DeepSeek-V4 attn_sink in the XPU
// sparse-MLA Triton kernel": the decode call site reads an fp8 cache; the
// Implementation paragraph gives the fold and the selected-only LSE).
//
// Cache layout (the page names the fp8 cache but not its encoding; this reads
// it in the plainest way): every latent row is 576 OCP fp8 e4m3 values (512
// latent + 64 rope, V = the first 512), with one fp32 scale per row, so the
// value is fp8(x) * kv_scale[row].
//
// Decode has few query rows, so each row's list is cut into nsplit pieces and
// every (row, 64-head group, piece) is its own workgroup (the partial kernel);
// a second kernel merges the pieces by their LSEs and folds the sink in once
// (the combine kernel, the same algebra as attn_sink_merge).  The partial
// results are fp32 in a caller-provided workspace, or, for the
// allocation-free entry point, in this file's static device scratch.
//
// Partial kernel, per 32-key tile: the 32 gathered fp8 rows (576 bytes each)
// go straight from memory into a 2-stage LDS ring (direct-to-LDS loads), are
// converted once to bf16 (exact: every e4m3 value is a bf16 value) into the
// line-major tile the bf16 prefill kernel reads, and then
//   S^T[key][head] = scale_k * (K[key] . Q[head])    (16x16x32 bf16 MFMAs)
//   O^T[dv][head] += V^T[dv][key] . (scale_k P)^T    (16x16x32 bf16 MFMAs)
// with the row scales of the tile held in LDS: the scale multiplies the logit
// and the probability that weights the row's V, never the bf16 operands.
#include "decode.hpp"

#include <mutex>

namespace attn {

namespace dec {
constexpr int DQK = 576, DV = 512;
constexpr int HPW = 16, NW = 4, HPB = HPW * NW;   // heads per wave / per workgroup
constexpr int KT = 32;                           // keys per tile
constexpr int ROWB = DQK;                        // fp8 bytes per latent row
constexpr int F8_TILE = KT * ROWB;               // 18 KB of fp8 per tile
constexpr int F8_LOADS = F8_TILE / 1024;         // 18 one-KB direct-to-LDS loads per tile
constexpr int TILE_EL = KT * DQK;                // bf16 elements of the converted tile
constexpr int CHUNK = 512;                       // list entries compacted per pass
constexpr int NQC = DQK / 32;
constexpr int NDV = DV / 16;
constexpr int KPIPE = 4, VPIPE = 4;
constexpr int CONV = DQK / 64;                   // 9 lines of 128 bf16 bytes per row
static_assert(F8_TILE % 1024 == 0 && KT * 8 == 256, "tile shapes: 8 threads per row");
}  // namespace dec

typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned dec_u32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 dec_bf16x2;

// 8 fp8 e4m3 bytes -> 8 bf16 (scale 1: exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(dec_u32x2 x) {
  const dec_bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false);
  const dec_bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true);
  const dec_bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false);
  const dec_bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int SINK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_fp8_partial(const DecodeParams p) {
  using namespace dec;
  __shared__ __attribute__((aligned(16))) unsigned char f8[2][F8_TILE];
  __shared__ __attribute__((aligned(16))) bf16 kt[TILE_EL];
  __shared__ __attribute__((aligned(16))) float sc[2][KT];
  __shared__ int kidx[CHUNK];
  __shared__ int wsum[NW];

  const int ngroups = p.Hq / HPB;
  const int b = blockIdx.x;                 // (row, head group), row-major
  const int split = blockIdx.y;
  const int i = b / ngroups;
  const int hg = b - i * ngroups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int h = hg * HPB + wave * HPW + col;

  const bf16* qrow = static_cast<const bf16*>(p.q) + (int64_t)i * p.q_row + (int64_t)h * p.q_head + 8 * grp;
  bf16x8 qf[NQC];
#pragma unroll
  for (int c = 0; c < NQC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);

  // bf16 tile layout (as in the prefill kernel): row r = 8 g + rr, 16-byte
  // chunk c = 8 L + c8 at byte (4 L + g) * 1024 + 128 rr + 16 (c8 ^ rr).
  const int rrk = col & 7;
  const int kofs_e = ((col >> 3) * 1024 + 128 * rrk + 16 * ((grp ^ rrk) & 7)) / 2;
  const int kofs_o = ((col >> 3) * 1024 + 128 * rrk + 16 * (((4 + grp) ^ rrk) & 7)) / 2;
  int vofs4[4];
  {
    const int rrv = 4 * (grp & 1) + (col >> 2), gv = grp >> 1, par = (col >> 1) & 1;
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
      vofs4[n4] = (gv * 1024 + 128 * rrv + 16 * (((2 * n4 + par) ^ rrv) & 7) + 8 * (col & 1)) / 2;
  }
  // fp8 -> bf16 conversion: thread (row cr = tid / 8, part cp = tid % 8)
  // converts bytes 8 (cp + 8 L) .. + 8 of its fp8 row (row-major, 576 B per
  // row) into 16-byte chunk cp of line L of the row in the bf16 tile, for the
  // 9 lines L; both addresses step by a constant per line.
  const int cr = tid >> 3, cpart = tid & 7;
  const int cv_src = cr * ROWB + 8 * cpart;
  const int cv_dst = ((cr >> 3) * 1024 + 128 * (cr & 7) + 16 * (cpart ^ (cr & 7))) / 2;
  auto convert = [&](int stage) {
#pragma unroll
    for (int L = 0; L < CONV; ++L) {
      const dec_u32x2 raw = *reinterpret_cast<const dec_u32x2*>(&f8[stage][cv_src + 64 * L]);
      *reinterpret_cast<bf16x8*>(kt + cv_dst + 2048 * L) = fp8x8_to_bf16(raw);
    }
  };

  const float sl2 = p.scale_log2;
  float m2 = kNegInf, lsum = 0.0f;
  floatx4 acc[NDV];
#pragma unroll
  for (int n = 0; n < NDV; ++n) acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int32_t* idx_row = p.topk_idx + (int64_t)i * p.topk_row;
  const int lo = split * p.split_len;
  const int hi = min(p.topk, lo + p.split_len);
  const unsigned char* kv = static_cast<const unsigned char*>(p.k);
  for (int c0 = lo; c0 < hi; c0 += CHUNK) {
    // ---- compact the valid entries of list[c0, min(c0 + CHUNK, hi)) into kidx[]
    __syncthreads();
    int mine[CHUNK / 256];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < CHUNK / 256; ++u) {
      const int e = c0 + tid * (CHUNK / 256) + u;
      const int j = e < hi ? idx_row[e] : -1;
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

    const int ntiles = (nvalid + KT - 1) / KT;
    // Tile t: the 18 one-KB pieces of its fp8 rows (piece q covers row-major
    // bytes 1024 q .. + 1024 of the tile; wave w issues pieces w, w + 4, ...),
    // and its 32 row scales into a register of wave 0.  Rows past the valid
    // count re-read a valid row (finite; their logits are masked).
    float sc_reg = 0.0f;
    auto issue = [&](int t, int stage) {
      // The per-load offsets are recomputed here from an opaque copy of the
      // lane id: hoisted out of the tile loop they are spilled, and reloading
      // a spilled offset waits for every vector load before it -- the
      // previous gathers of the tile -- so the gathers ran one at a time.
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int k = 0; k < (F8_LOADS + NW - 1) / NW; ++k) {
        const int q = wave + NW * k;
        if (q < F8_LOADS) {  // wave-uniform
          const int byte = 1024 * q + 16 * ln;
          const int r = byte / ROWB, off = byte - r * ROWB;
          const int posr = t * KT + r;
          const int j = kidx[posr < nvalid ? posr : 0];
          load_lds16_m0(kv + (int64_t)j * p.k_row + off, lds_addr(&f8[stage][0]) + 1024 * q);
        }
      }
      if (wave == 0 && lane < KT) {
        const int posr = t * KT + lane;
        sc_reg = p.kv_scale[kidx[posr < nvalid ? posr : 0]];
      }
    };

    auto compute = [&](int t, int stage) {
      const int t0 = t * KT;
      float s[2][4];
      floatx4 scv[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) scv[sb] = *reinterpret_cast<const floatx4*>(&sc[stage][16 * sb + 4 * grp]);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
        const bf16* krow = kt + 1024 * sb;
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
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[sb][e] = (t0 + 16 * sb + 4 * grp + e < nvalid) ? a[e] * (sl2 * scv[sb][e]) : kNegInf;
      }
      float mt = kNegInf;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mt = fmaxf(mt, s[sb][e]);
      // the lanes' maxima are exchanged only on the rescale path: a column
      // passes the threshold iff one of its lanes does
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
          pb[4 * sb + e] = static_cast<bf16>(pe * scv[sb][e]);  // the row scale weights V
        }
      lsum += ps;
      auto vload = [&](int n) {
        const bf16* v0 = kt + vofs4[n & 3] + 2048 * (n >> 2);
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

    if (ntiles > 0) issue(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      const int stage = t & 1;
      wait_vmcnt<0>();                      // tile t's fp8 rows and scales have landed
      if (wave == 0 && lane < KT) sc[stage][lane] = sc_reg;
      lds_barrier();                        // every wave is done with tile t - 1
      if (t + 1 < ntiles) issue(t + 1, stage ^ 1);
      convert(stage);
      lds_barrier();                        // the bf16 tile and its scales are in place
      compute(t, stage);
    }
  }

  // ---- partial result of this piece: out normalised by its own sum, LSE
  lsum = sum_over_groups(lsum);
  const float f = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  float* po = p.ws_out + (((int64_t)split * p.T + i) * p.Hq + h) * DV + 4 * grp;
#pragma unroll
  for (int n = 0; n < NDV; ++n) {
    floatx4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = acc[n][e] * f;
    *reinterpret_cast<floatx4*>(po + 16 * n) = o;
  }
  if (grp == 0) p.ws_lse[((int64_t)split * p.Hq + h) * p.T + i] = lse_natural(m2, lsum);
}

// Merge of the nsplit partials of every (row, head) by their LSEs, then the
// null-logit sink: out = sum_s e^{lse_s - lse} out_s / (1 + e^{sink - lse}),
// lse = log sum_s e^{lse_s} (selected keys only).  One lane per 8 outputs.
template <int SINK>
__global__ __launch_bounds__(256) void mla_decode_fp8_combine(const DecodeParams p) {
  constexpr int DV = dec::DV, CPR = DV / 8;
  const int64_t total = (int64_t)p.T * p.Hq * CPR;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
    const int64_t rh = c / CPR;
    const int d = (int)(c - rh * CPR);
    const int i = (int)(rh / p.Hq), h = (int)(rh - (int64_t)i * p.Hq);
    float m = kNegInf;
    for (int s = 0; s < p.nsplit; ++s) m = fmaxf(m, p.ws_lse[((int64_t)s * p.Hq + h) * p.T + i]);
    float acc[8] = {};
    float lse = kNegInf;
    if (m != kNegInf) {
      float wsum = 0.0f;
      for (int s = 0; s < p.nsplit; ++s) {
        const float w = expf(p.ws_lse[((int64_t)s * p.Hq + h) * p.T + i] - m);
        wsum += w;
        const float* src = p.ws_out + (((int64_t)s * p.T + i) * p.Hq + h) * DV + 8 * d;
        const floatx4 a = *reinterpret_cast<const floatx4*>(src);
        const floatx4 b = *reinterpret_cast<const floatx4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] = __builtin_fmaf(w, a[e], acc[e]);
          acc[4 + e] = __builtin_fmaf(w, b[e], acc[4 + e]);
        }
      }
      lse = m + logf(wsum);
      float f = 1.0f / wsum;
      if (SINK == kSinkNull) f = f / (1.0f + expf(p.sinks[h] - lse));
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= f;
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<bf16>(acc[e]);
    *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + (int64_t)i * p.o_row + (int64_t)h * p.o_head + 8 * d) = o;
    if (d == 0) p.lse[(int64_t)h * p.T + i] = lse;
  }
}

// ---------------------------------------------------------------- scratch of the allocation-free entry point
// The partial results of attn_sink_mla_decode_fp8_noalloc live in this
// file-scope device array (one copy per GPU, held for the life of the
// process).  On the host `scratch` only names the symbol: its device address
// is looked up once per device with hipGetSymbolAddress and that address is
// what the kernels receive.  Every call on a GPU shares its copy; calls that
// overlap on one GPU race.  Nothing in it needs to start at zero: the partial
// kernel writes every (piece, row, head) slot before the combine reads it.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {  // first call on this device, with it current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

int decode_splits(int64_t T, int64_t Hq, int64_t topk) {
  const int64_t wgs = T * (Hq / dec::HPB);
  const int64_t max_split = (topk + dec::KT - 1) / dec::KT;  // at least one tile per piece
  int64_t s = wgs > 0 ? (512 + wgs - 1) / wgs : 1;  // about two workgroups per CU
  if (s > max_split) s = max_split;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

int decode_split_len(int64_t topk, int nsplit) {
  const int64_t per = (topk + nsplit - 1) / nsplit;
  return (int)(((per + dec::KT - 1) / dec::KT) * dec::KT);
}

hipError_t launch_mla_decode_fp8(const DecodeParams& p, int sink, hipStream_t st) {
  const dim3 grid1((unsigned)((int64_t)p.T * (p.Hq / dec::HPB)), (unsigned)p.nsplit), block(256);
  const int64_t chunks = (int64_t)p.T * p.Hq * (dec::DV / 8);
  const dim3 grid2((unsigned)((chunks + 255) / 256 < 8192 ? (chunks + 255) / 256 : 8192));
  if (sink == kSinkNull) {
    hipLaunchKernelGGL(mla_decode_fp8_partial<kSinkNull>, grid1, block, 0, st, p);
    hipLaunchKernelGGL(mla_decode_fp8_combine<kSinkNull>, grid2, block, 0, st, p);
  } else {
    hipLaunchKernelGGL(mla_decode_fp8_partial<kSinkNone>, grid1, block, 0, st, p);
    hipLaunchKernelGGL(mla_decode_fp8_combine<kSinkNone>, grid2, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace attn
