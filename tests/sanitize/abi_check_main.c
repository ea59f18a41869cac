/* Host-side validation of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every call here is a *_check entry point (or
 * an entry point whose arguments make it return before any launch), so no
 * GPU is needed; data pointers are placeholders that are never dereferenced.
 * The program exits non-zero on the first unexpected status; the sanitizers
 * abort on any invalid memory access or undefined operation. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn_sink.h"

static int failures = 0;
#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    int rc_ = (call);                                                                  \
    if (rc_ != (want)) {                                                               \
      fprintf(stderr, "%s:%d: %s returned %d, want %d\n", __FILE__, __LINE__, #call,   \
              rc_, (int)(want));                                                       \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

static void* const FAKE = (void*)(uintptr_t)0x100000; /* 16-byte aligned, never touched */

static attn_tensor dense(int dtype, int ndim, const int64_t* shape) {
  attn_tensor t;
  memset(&t, 0, sizeof t);
  t.data = FAKE;
  t.dtype = dtype;
  t.ndim = ndim;
  int64_t acc = 1;
  for (int d = ndim - 1; d >= 0; --d) {
    t.shape[d] = shape[d];
    t.stride[d] = acc;
    acc *= shape[d];
  }
  return t;
}

static void window_calls(void) {
  const int64_t T = 300, Hq = 16, Hkv = 4;
  const int64_t D[] = {64, 80, 96, 128};
  const int32_t* cu = (const int32_t*)FAKE;
  const float* sinks = (const float*)FAKE;
  float* lse = (float*)FAKE;
  for (int di = 0; di < 4; ++di) {
    int64_t sq[3] = {T, Hq, D[di]}, sk[3] = {T, Hkv, D[di]};
    attn_tensor q = dense(ATTN_DTYPE_BF16, 3, sq), k = dense(ATTN_DTYPE_BF16, 3, sk);
    attn_tensor v = k, o = q;
    for (int32_t W = -1; W <= 70; W += 71) {
      for (int sm = -1; sm <= 3; ++sm) {
        attn_mask_arg m = {W, 0, NULL, NULL};
        int want = (sm < 0 || sm > 2) ? ATTN_ERR_ENUM : (W < 0 ? ATTN_ERR_RANGE : ATTN_OK);
        EXPECT(attn_sink_check(&q, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, sm, 0.1f, &o, lse), want);
      }
    }
    attn_mask_arg wide = {INT32_MAX, 0, NULL, NULL};
    EXPECT(attn_sink_check(&q, &k, &v, cu, 3, ATTN_MASK_WINDOW, &wide, sinks, ATTN_SINK_KEY0_BIAS, 0.1f, &o, lse),
           ATTN_OK);
    attn_tensor f = q, fk = k;
    f.dtype = ATTN_DTYPE_F32;
    fk.dtype = ATTN_DTYPE_F32;
    EXPECT(attn_sink_check(&f, &fk, &fk, cu, 3, ATTN_MASK_WINDOW, &wide, sinks, ATTN_SINK_NULL_LOGIT, 0.1f, &f, lse),
           ATTN_OK);
    /* mismatches of every kind */
    attn_mask_arg m = {8, 0, NULL, NULL};
    EXPECT(attn_sink_check(NULL, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_NULL);
    EXPECT(attn_sink_check(&q, &k, &v, NULL, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_NULL);
    EXPECT(attn_sink_check(&q, &k, &v, cu, 0, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_RANGE);
    EXPECT(attn_sink_check(&q, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, NULL, 1, 0.1f, &o, lse), ATTN_ERR_NULL);
    EXPECT(attn_sink_check(&q, &k, &v, cu, 3, 7, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_ENUM);
    attn_tensor bad = q;
    bad.stride[2] = 2;
    EXPECT(attn_sink_check(&bad, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_STRIDE);
    bad = q;
    bad.shape[0] = T + 1;
    EXPECT(attn_sink_check(&bad, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_SHAPE);
    bad = k;
    bad.shape[1] = 3;
    attn_tensor badv = bad;
    EXPECT(attn_sink_check(&q, &bad, &badv, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_HEADS);
    bad = q;
    bad.ndim = 5; /* out of the descriptor's range: must be refused, never indexed */
    EXPECT(attn_sink_check(&bad, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_SHAPE);
    bad = q;
    bad.dtype = 99;
    EXPECT(attn_sink_check(&bad, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, 0.1f, &o, lse), ATTN_ERR_ENUM);
    float nan;
    uint32_t bits = 0x7fc00000u;
    memcpy(&nan, &bits, 4);
    EXPECT(attn_sink_check(&q, &k, &v, cu, 3, ATTN_MASK_WINDOW, &m, sinks, 1, nan, &o, lse), ATTN_ERR_RANGE);
  }
  /* huge grids are refused by the check */
  int64_t hq[3] = {INT32_MAX, 2, 64}, hk[3] = {INT32_MAX, 1, 64};
  attn_tensor q = dense(ATTN_DTYPE_BF16, 3, hq), k = dense(ATTN_DTYPE_BF16, 3, hk);
  attn_mask_arg m = {4, 0, NULL, NULL};
  EXPECT(attn_sink_check(&q, &k, &k, cu, 1, ATTN_MASK_WINDOW, &m, NULL, 0, 0.1f, &q, lse), ATTN_ERR_RANGE);
  /* T = 0 returns before any launch, also from the launching entry point */
  int64_t z[3] = {0, 4, 64}, zk[3] = {0, 4, 64};
  attn_tensor zq = dense(ATTN_DTYPE_BF16, 3, z), zkv = dense(ATTN_DTYPE_BF16, 3, zk);
  zq.data = NULL;
  zkv.data = NULL;
  EXPECT(attn_sink_fwd(&zq, &zkv, &zkv, cu, 1, ATTN_MASK_WINDOW, &m, NULL, 0, 0.1f, &zq, NULL, 0), ATTN_OK);
}

static void topk_and_blocksel_calls(void) {
  const float* sinks = (const float*)FAKE;
  float* lse = (float*)FAKE;
  int64_t sq[3] = {8, 64, 576}, skv[3] = {100, 1, 576}, so[3] = {8, 64, 512}, si[2] = {8, 16};
  attn_tensor q = dense(ATTN_DTYPE_BF16, 3, sq), kv = dense(ATTN_DTYPE_BF16, 3, skv);
  attn_tensor v = kv, o = dense(ATTN_DTYPE_BF16, 3, so), idx = dense(ATTN_DTYPE_I32, 2, si);
  v.shape[2] = 512;
  attn_mask_arg m = {0, 0, &idx, NULL};
  EXPECT(attn_sink_check(&q, &kv, &v, NULL, 0, ATTN_MASK_TOPK, &m, sinks, ATTN_SINK_NULL_LOGIT, 0.04f, &o, lse), ATTN_OK);
  EXPECT(attn_sink_check(&q, &kv, &v, NULL, 0, ATTN_MASK_TOPK, &m, sinks, ATTN_SINK_KEY0_BIAS, 0.04f, &o, lse),
         ATTN_ERR_UNSUPPORTED);
  attn_mask_arg none = {0, 0, NULL, NULL};
  EXPECT(attn_sink_check(&q, &kv, &v, NULL, 0, ATTN_MASK_TOPK, &none, sinks, 2, 0.04f, &o, lse), ATTN_ERR_NULL);
  idx.dtype = ATTN_DTYPE_I64;
  EXPECT(attn_sink_check(&q, &kv, &v, NULL, 0, ATTN_MASK_TOPK, &m, sinks, 2, 0.04f, &o, lse), ATTN_ERR_DTYPE);

  int64_t T = 300, NB = 5;
  int64_t bq[3] = {T, 32, 128}, bk[3] = {T, 8, 128}, bt[4] = {1, 8, T, NB};
  attn_tensor Q = dense(ATTN_DTYPE_BF16, 3, bq), K = dense(ATTN_DTYPE_BF16, 3, bk), B = dense(ATTN_DTYPE_U8, 4, bt);
  attn_mask_arg bm = {0, 64, NULL, &B};
  const int32_t* cu = (const int32_t*)FAKE;
  for (int sm = 0; sm <= 2; ++sm)
    EXPECT(attn_sink_check(&Q, &K, &K, cu, 2, ATTN_MASK_BLOCKSEL, &bm, sinks, sm, 0.088f, &Q, lse), ATTN_OK);
  B.shape[3] = NB - 1;
  EXPECT(attn_sink_check(&Q, &K, &K, cu, 2, ATTN_MASK_BLOCKSEL, &bm, sinks, 0, 0.088f, &Q, lse), ATTN_ERR_SHAPE);
  B.shape[3] = NB;
  B.shape[1] = 3;
  EXPECT(attn_sink_check(&Q, &K, &K, cu, 2, ATTN_MASK_BLOCKSEL, &bm, sinks, 0, 0.088f, &Q, lse), ATTN_ERR_HEADS);
  B.shape[1] = 8;
  bm.block_size = 0;
  EXPECT(attn_sink_check(&Q, &K, &K, cu, 2, ATTN_MASK_BLOCKSEL, &bm, sinks, 0, 0.088f, &Q, lse), ATTN_ERR_RANGE);
}

static void compose_cp_decode_calls(void) {
  const float* sinks = (const float*)FAKE;
  float* lse = (float*)FAKE;
  int64_t so[3] = {64, 8, 128};
  attn_tensor parts[ATTN_SINK_MERGE_MAX_PARTS + 1];
  const float* plse[ATTN_SINK_MERGE_MAX_PARTS + 1];
  for (int i = 0; i <= ATTN_SINK_MERGE_MAX_PARTS; ++i) {
    parts[i] = dense(ATTN_DTYPE_BF16, 3, so);
    parts[i].data = (char*)FAKE + 0x100000 * (i + 1);
    plse[i] = (const float*)((char*)FAKE + 0x100000 * (i + 1) + 0x80000);
  }
  attn_tensor out = dense(ATTN_DTYPE_BF16, 3, so);
  for (int n = 0; n <= ATTN_SINK_MERGE_MAX_PARTS + 1; ++n) {
    int want = (n < 1 || n > ATTN_SINK_MERGE_MAX_PARTS) ? ATTN_ERR_RANGE : ATTN_OK;
    EXPECT(attn_sink_merge_check(parts, plse, n, sinks, ATTN_SINK_NULL_LOGIT, &out, lse), want);
  }
  EXPECT(attn_sink_merge_check(parts, plse, 2, sinks, ATTN_SINK_KEY0_BIAS, &out, lse), ATTN_ERR_UNSUPPORTED);

  int64_t wq[3] = {200, 4, 64};
  attn_tensor q = dense(ATTN_DTYPE_BF16, 3, wq);
  const int32_t* cu = (const int32_t*)FAKE;
  EXPECT(attn_sink_key0_correct_check(&q, &q, &q, cu, 2, 16, sinks, 0.1f, &q, lse), ATTN_OK);
  EXPECT(attn_sink_key0_correct_check(&q, &q, &q, cu, 2, INT32_MAX, sinks, 0.1f, &q, lse), ATTN_OK);
  EXPECT(attn_sink_key0_correct_check(&q, &q, &q, cu, 2, -1, sinks, 0.1f, &q, lse), ATTN_ERR_RANGE);

  int64_t* slots = (int64_t*)FAKE;
  EXPECT(attn_sink_cp_slots_check(8, 64, -1, slots), ATTN_OK);
  EXPECT(attn_sink_cp_slots_check(8, 63, 0, slots), ATTN_ERR_RANGE);
  EXPECT(attn_sink_cp_slots_check(8, 64, 8, slots), ATTN_ERR_RANGE);
  int64_t rs[2] = {100, 256}, rd[2] = {100, 256};
  attn_tensor src = dense(ATTN_DTYPE_BF16, 2, rs), dst = dense(ATTN_DTYPE_BF16, 2, rd);
  dst.data = (char*)FAKE + 0x200000;
  EXPECT(attn_sink_cp_permute_rows_check(&src, slots, 100, 1, &dst), ATTN_OK);
  EXPECT(attn_sink_cp_permute_rows_check(&src, slots, 100, 2, &dst), ATTN_ERR_ENUM);
  EXPECT(attn_sink_cp_permute_rows_check(&src, slots, 100, 0, &src), ATTN_ERR_RANGE);
  int32_t* i32 = (int32_t*)FAKE;
  EXPECT(attn_sink_cp_documents_check(slots, 1000, i32, i32, 8, i32), ATTN_OK);
  EXPECT(attn_sink_cp_documents_check(slots, -1, i32, i32, 8, i32), ATTN_ERR_RANGE);

  int64_t bytes = -1;
  EXPECT(attn_sink_mla_decode_fp8_workspace(128, 64, 2048, &bytes), ATTN_OK);
  if (bytes <= 0) ++failures;
  EXPECT(attn_sink_mla_decode_fp8_workspace(128, 63, 2048, &bytes), ATTN_ERR_RANGE);
  EXPECT(attn_sink_mla_decode_fp8_workspace(128, 64, 2048, NULL), ATTN_ERR_NULL);
  int64_t dq[3] = {128, 64, 576}, dkv[3] = {1000, 1, 576}, dout[3] = {128, 64, 512}, di[2] = {128, 2048};
  attn_tensor Q = dense(ATTN_DTYPE_BF16, 3, dq), KV = dense(ATTN_DTYPE_FP8_E4M3, 3, dkv);
  attn_tensor O = dense(ATTN_DTYPE_BF16, 3, dout), I = dense(ATTN_DTYPE_I32, 2, di);
  EXPECT(attn_sink_mla_decode_fp8_workspace(128, 64, 2048, &bytes), ATTN_OK);
  EXPECT(attn_sink_mla_decode_fp8_check(&Q, &KV, sinks, &I, sinks, 2, 0.04f, &O, lse, FAKE, bytes), ATTN_OK);
  EXPECT(attn_sink_mla_decode_fp8_check(&Q, &KV, sinks, &I, sinks, 2, 0.04f, &O, lse, FAKE, bytes - 1),
         ATTN_ERR_RANGE);
  for (int s = -20; s <= 20; ++s) {
    const char* msg = attn_sink_strerror(s);
    if (!msg || !msg[0]) ++failures;
  }
}

int main(void) {
  window_calls();
  topk_and_blocksel_calls();
  compose_cp_decode_calls();
  if (failures) {
    fprintf(stderr, "%d unexpected status codes\n", failures);
    return 1;
  }
  printf("abi checks: all statuses as expected\n");
  return 0;
}
