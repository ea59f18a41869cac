/* The C oracle (oracle/ref.c) on small inputs of every mask kind and sink
 * mode under AddressSanitizer and UndefinedBehaviorSanitizer: every read of
 * q, k, v, cu_seqlens, the index lists and the selection table must stay in
 * bounds, including padding entries, out-of-range indices, empty rows, row
 * subsets and an unbounded window.  A few results with a plain closed form
 * are checked too (constant values, the -inf null sink). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_fwd(const float* q, const float* k, const float* v, int64_t T, int64_t Tk, int Hq, int Hkv,
                    int Dqk, int Dv, const int32_t* cu_seqlens, int num_seqs, int mask_kind, int window,
                    const int32_t* topk_idx, int topk, const uint8_t* block_sel, int Hidx, int NB,
                    int block_size, const double* sinks, int sink_mode, double scale, const int64_t* rows,
                    int64_t nrows, double* out, double* lse);

static int failures = 0;
static uint32_t state = 12345u;
static float rnd(void) {
  state = state * 1664525u + 1013904223u;
  return ((int32_t)(state >> 8) - (1 << 23)) / (float)(1 << 23);
}

/* exact-size heap copies, so that any read past the end is caught */
static void* dup(const void* p, size_t n) {
  void* d = malloc(n ? n : 1);
  memcpy(d, p, n);
  return d;
}

static void run(int mask_kind, int sink_mode, int window, int use_rows, int const_v) {
  enum { T = 37, Hq = 4, Hkv = 2, D = 16, DV = 8, TOPK = 9, BS = 4 };
  const int NB = (T + BS - 1) / BS;
  float qb[T * Hq * D], kb[T * Hkv * D], vb[T * Hkv * DV];
  for (int i = 0; i < T * Hq * D; ++i) qb[i] = rnd();
  for (int i = 0; i < T * Hkv * D; ++i) kb[i] = rnd();
  for (int i = 0; i < T * Hkv * DV; ++i) vb[i] = const_v ? 0.75f : rnd();
  int32_t cub[4] = {0, 5, 5, T};                       /* an empty segment in the middle */
  int32_t idxb[T * TOPK];
  for (int i = 0; i < T * TOPK; ++i) {
    int r = (int)(state % 7u);
    rnd();
    idxb[i] = r == 0 ? -1 : r == 1 ? T + 3 : r == 2 ? -1000 : (int32_t)(state % (uint32_t)T);
  }
  for (int i = 0; i < TOPK; ++i) idxb[5 * TOPK + i] = -1;   /* an all-padding row: empty */
  uint8_t tabb[1 * 2 * T * 10];
  for (int i = 0; i < 2 * T * NB; ++i) { rnd(); tabb[i] = (state >> 29) & 1; }
  memset(tabb + 7 * NB, 0, NB);                              /* an all-zero table row: empty */
  double sk[Hq] = {0.3, -1.5, 2.0, -INFINITY};
  int64_t rowsb[5] = {36, 0, 5, 17, 5};

  float* q = dup(qb, sizeof qb);
  float* k = dup(kb, sizeof kb);
  float* v = dup(vb, sizeof vb);
  int32_t* cu = dup(cub, sizeof cub);
  int32_t* idx = dup(idxb, sizeof idxb);
  uint8_t* tab = dup(tabb, (size_t)2 * T * NB);
  double* sinks = dup(sk, sizeof sk);
  int64_t* rows = dup(rowsb, sizeof rowsb);
  const int64_t nrows = use_rows ? 5 : T;
  double* out = malloc(sizeof(double) * (size_t)nrows * Hq * DV);
  double* lse = malloc(sizeof(double) * (size_t)nrows * Hq);
  int rc = oracle_attn_fwd(q, k, v, T, T, Hq, Hkv, D, DV, cu, 3, mask_kind, window, idx, TOPK, tab, 2, NB, BS,
                           sink_mode ? sinks : NULL, sink_mode, 0.25, use_rows ? rows : NULL, nrows, out, lse);
  if (rc != 0) {
    fprintf(stderr, "oracle rejected mask %d sink %d\n", mask_kind, sink_mode);
    ++failures;
  }
  for (int64_t r = 0; r < nrows && rc == 0; ++r)
    for (int h = 0; h < Hq; ++h) {
      const double l = lse[(int64_t)h * nrows + r];
      for (int d = 0; d < DV; ++d) {
        const double o = out[(r * Hq + h) * DV + d];
        if (isinf(l) && o != 0.0) ++failures;            /* empty rows are zero */
        if (!isinf(l) && const_v && sink_mode != 2 && fabs(o - 0.75) > 1e-12) ++failures;
        if (!isinf(l) && const_v && sink_mode == 2 && h == 3 && fabs(o - 0.75) > 1e-12) ++failures;
      }
    }
  free(q); free(k); free(v); free(cu); free(idx); free(tab); free(sinks); free(rows); free(out); free(lse);
}

int main(void) {
  const int windows[4] = {0, 3, 40, 2147483647};
  for (int sm = 0; sm <= 2; ++sm)
    for (int cv = 0; cv <= 1; ++cv)
      for (int ur = 0; ur <= 1; ++ur) {
        for (int w = 0; w < 4; ++w) run(0, sm, windows[w], ur, cv);
        if (sm != 1) run(1, sm, 0, ur, cv);
        run(2, sm, 0, ur, cv);
      }
  /* argument errors are reported, not dereferenced */
  double o[8], l[1];
  float x[16];
  int32_t cu[2] = {0, 1};
  if (oracle_attn_fwd(NULL, x, x, 1, 1, 1, 1, 16, 8, cu, 1, 0, 1, NULL, 0, NULL, 0, 0, 0, NULL, 0, 1.0, NULL, 1, o, l) != -1)
    ++failures;
  if (oracle_attn_fwd(x, x, x, 1, 1, 1, 1, 16, 8, NULL, 1, 0, 1, NULL, 0, NULL, 0, 0, 0, NULL, 0, 1.0, NULL, 1, o, l) != -1)
    ++failures;
  if (oracle_attn_fwd(x, x, x, 1, 1, 1, 1, 16, 8, cu, 1, 1, 0, NULL, 4, NULL, 0, 0, 0, NULL, 0, 1.0, NULL, 1, o, l) != -1)
    ++failures;
  if (failures) {
    fprintf(stderr, "%d oracle checks failed\n", failures);
    return 1;
  }
  printf("oracle: all cases clean\n");
  return 0;
}
