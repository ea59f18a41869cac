/*
 * Plain fp64 CPU oracle for sink-aware masked attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the benchmark's
 * CPU-baseline leg can compare the HIP kernels against an independent,
 * obviously-correct implementation.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (the plain definition, written out key by key):
 *   For every query row i and query head h (kv head = h / (Hq/Hkv)):
 *     S(i,h)  = the valid key set of row i (see the three mask kinds below)
 *     l_j     = scale * sum_d q[i,h,d] * k[j,kv,d]                for j in S
 *     key0_bias: l_j += sinks[h] when j is the first key of its cu_seqlens
 *                segment ("[Bugfix][MiMo] Apply vision attention sinks in the
 *                window attention path", closed-form correction paragraph: the
 *                per-head sink biases key 0 of every sequence; it enters the
 *                already-scaled logit, since that correction multiplies key
 *                0's softmax weight by exp(s)).
 *     empty S: out = 0, lse = -inf ("cp_sparse_attn" API page,
 *              _local_sparse_forward: fully masked rows give zero output).
 *     m = max l_j, Z = sum exp(l_j - m), A = sum exp(l_j - m) * v[j,kv,:]
 *     none / key0_bias: out = A / Z
 *     null_logit:       out = A / (Z + exp(sinks[h] - m))
 *                       ("Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA
 *                       Triton kernel", Implementation paragraph: the sink
 *                       joins the softmax denominator only)
 *     lse = m + log(Z)  (natural log over the selected keys only; the
 *                        null-logit sink never enters it, same paragraph)
 *
 * Mask kinds:
 *   window   (mask_kind 0): j in the same cu_seqlens segment as i and
 *            |i - j| <= W.  The bound is inclusive: on the MiMo page the rows
 *            that reach key 0 are the sequence's first W + 1 (rows 0 .. W).
 *   topk     (mask_kind 1): j = topk_idx[i, t] for every t with
 *            0 <= topk_idx[i, t] < Tk; -1 (or anything outside) is padding.
 *            The list is shared by all heads (sparse MLA with one latent KV).
 *   blocksel (mask_kind 2): block_sel[0, h / (Hq/Hidx), i, j / block_size]
 *            != 0, and j <= i (token causal), and j in the same cu_seqlens
 *            segment (document) as i.  Table offsets are 64-bit: the
 *            "cp_sparse_attn" page, _block_sel_flat_offset, shows a 32-bit
 *            flat offset wrapping past 2**31 table elements.
 *
 * Inputs are float32 arrays holding the exact values the GPU reads (bf16
 * inputs are exactly representable in float32); every product and sum is
 * taken in double.  Layouts are dense row-major: q[T][Hq][Dqk],
 * k[Tk][Hkv][Dqk], v[Tk][Hkv][Dv], out[nrows][Hq][Dv], lse[Hq][nrows].
 * `rows` (optional) lists the query rows to evaluate; outputs are compacted
 * in that order.  Parallel over (row, head) with OpenMP; no blocking, no
 * reordering of the per-row sums beyond the definition above.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_WINDOW = 0, ORC_TOPK = 1, ORC_BLOCKSEL = 2 };
enum { ORC_SINK_NONE = 0, ORC_SINK_KEY0_BIAS = 1, ORC_SINK_NULL_LOGIT = 2 };

/* 64-bit flat offset of [b, h, q, kb] in a [B, H, S, NB] table. */
int64_t oracle_blocksel_offset(int64_t b, int64_t h, int64_t q, int64_t kb,
                               int64_t H, int64_t S, int64_t NB) {
  return ((b * H + h) * S + q) * NB + kb;
}

/* Segment (sequence / document) index of token t: the s with
 * cu[s] <= t < cu[s+1].  Linear scan: plain and obviously right. */
static int segment_of(const int32_t* cu, int num_seqs, int64_t t) {
  for (int s = 0; s < num_seqs; ++s)
    if (cu[s] <= t && t < cu[s + 1]) return s;
  return -1;
}

/* Collect S(i,h) into keys[]; returns |S|. */
static int64_t key_set(int mask_kind, int64_t i, int h, int64_t Tk, int Hq,
                       const int32_t* cu, int num_seqs, int window,
                       const int32_t* topk_idx, int topk,
                       const uint8_t* block_sel, int Hidx, int64_t T, int NB,
                       int block_size, int64_t* keys) {
  int64_t n = 0;
  if (mask_kind == ORC_WINDOW) {
    int s = segment_of(cu, num_seqs, i);
    if (s < 0) return 0;
    for (int64_t j = cu[s]; j < cu[s + 1]; ++j) {
      int64_t d = i > j ? i - j : j - i;
      if (d <= window) keys[n++] = j;
    }
  } else if (mask_kind == ORC_TOPK) {
    for (int t = 0; t < topk; ++t) {
      int64_t j = topk_idx[i * (int64_t)topk + t];
      if (j >= 0 && j < Tk) keys[n++] = j;
    }
  } else {
    int s = segment_of(cu, num_seqs, i);
    if (s < 0) return 0;
    int hidx = h / (Hq / Hidx);
    for (int64_t j = cu[s]; j <= i; ++j) {
      int64_t off = oracle_blocksel_offset(0, hidx, i, j / block_size, Hidx, T, NB);
      if (block_sel[off]) keys[n++] = j;
    }
  }
  return n;
}

/* Returns 0 on success, -1 on a bad argument. */
int oracle_attn_fwd(const float* q, const float* k, const float* v,
                    int64_t T, int64_t Tk, int Hq, int Hkv, int Dqk, int Dv,
                    const int32_t* cu_seqlens, int num_seqs,
                    int mask_kind, int window,
                    const int32_t* topk_idx, int topk,
                    const uint8_t* block_sel, int Hidx, int NB, int block_size,
                    const double* sinks, int sink_mode, double scale,
                    const int64_t* rows, int64_t nrows,
                    double* out, double* lse) {
  if (!q || !k || !v || !out || !lse || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return -1;
  if (mask_kind == ORC_TOPK && (!topk_idx || sink_mode == ORC_SINK_KEY0_BIAS)) return -1;
  if (mask_kind != ORC_TOPK && (!cu_seqlens || num_seqs <= 0)) return -1;
  if (mask_kind == ORC_BLOCKSEL && (!block_sel || Hidx <= 0 || Hq % Hidx || block_size <= 0)) return -1;
  if (sink_mode != ORC_SINK_NONE && !sinks) return -1;
  if (rows == NULL) nrows = T;
  const int g = Hq / Hkv;
  int64_t maxkeys = mask_kind == ORC_TOPK ? topk : (mask_kind == ORC_WINDOW ? 2 * (int64_t)window + 1 : Tk);
  if (maxkeys > Tk && mask_kind != ORC_TOPK) maxkeys = Tk;
  int failed = 0;

#pragma omp parallel
  {
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(maxkeys > 0 ? maxkeys : 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)(maxkeys > 0 ? maxkeys : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)Dv);
    if (!keys || !logit || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < nrows * Hq; ++r) {
        int64_t ri = r / Hq;
        int h = (int)(r % Hq);
        int64_t i = rows ? rows[ri] : ri;
        int kv = h / g;
        double* o = out + (ri * Hq + h) * (int64_t)Dv;
        int64_t n = key_set(mask_kind, i, h, Tk, Hq, cu_seqlens, num_seqs, window,
                            topk_idx, topk, block_sel, Hidx, T, NB, block_size, keys);
        if (n == 0) {
          for (int d = 0; d < Dv; ++d) o[d] = 0.0;
          lse[(int64_t)h * nrows + ri] = -INFINITY;
          continue;
        }
        const float* qi = q + (i * Hq + h) * (int64_t)Dqk;
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
          int64_t j = keys[t];
          const float* kj = k + (j * Hkv + kv) * (int64_t)Dqk;
          double dot = 0.0;
          for (int d = 0; d < Dqk; ++d) dot += (double)qi[d] * (double)kj[d];
          double l = scale * dot;
          if (sink_mode == ORC_SINK_KEY0_BIAS) {
            int s = segment_of(cu_seqlens, num_seqs, j);
            if (s >= 0 && j == cu_seqlens[s]) l += sinks[h];
          }
          logit[t] = l;
          if (l > m) m = l;
        }
        double Z = 0.0;
        for (int d = 0; d < Dv; ++d) acc[d] = 0.0;
        for (int64_t t = 0; t < n; ++t) {
          double p = exp(logit[t] - m);
          const float* vj = v + (keys[t] * Hkv + kv) * (int64_t)Dv;
          Z += p;
          for (int d = 0; d < Dv; ++d) acc[d] += p * (double)vj[d];
        }
        double denom = Z;
        if (sink_mode == ORC_SINK_NULL_LOGIT) denom = Z + exp(sinks[h] - m);
        for (int d = 0; d < Dv; ++d) o[d] = acc[d] / denom;
        lse[(int64_t)h * nrows + ri] = m + log(Z);
      }
    }
    free(keys);
    free(logit);
    free(acc);
  }
  return failed ? -1 : 0;
}

/* Threads the OpenMP runtime will use (for reporting the CPU baseline). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
