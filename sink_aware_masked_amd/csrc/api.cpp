// C ABI front end: argument validation, kernel-instance selection and a single
// launch on the caller's stream.  No allocation, no synchronisation, no device
// reads from the host.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "attn_sink.h"
#include "common.hpp"
#include "compose.hpp"
#include "cp.hpp"
#include "decode.hpp"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace attn {
hipError_t launch_window_bf16(const Params& p, int sink, hipStream_t st);
hipError_t launch_generic_f32(const Params& p, int mask, int sink, hipStream_t st);
hipError_t launch_topk_mla_bf16(const Params& p, int sink, hipStream_t st);
hipError_t launch_blocksel_bf16(const Params& p, int sink, hipStream_t st);
int64_t window_bf16_items(const Params& p);
int64_t generic_f32_items(const Params& p);
int64_t topk_mla_bf16_items(const Params& p);
int64_t blocksel_bf16_items(const Params& p);
}  // namespace attn

static_assert(attn::kMergeMaxParts == ATTN_SINK_MERGE_MAX_PARTS, "merge part limit");

namespace {

using attn::Params;

enum Instance { kInstNone = 0, kInstGenericF32, kInstWindowBf16, kInstTopkMlaBf16, kInstBlockselBf16 };

constexpr int64_t kMaxTokens = 0x7fffffffLL;
// A launch's x dimension holds at most 2^32 - 1 work items (workgroups times
// workgroup size); calls whose grid would exceed it are refused up front.
constexpr int64_t kMaxGridItems = 0xffffffffLL;

int elem_size(int32_t dt) {
  switch (dt) {
    case ATTN_DTYPE_BF16: return 2;
    case ATTN_DTYPE_F32: return 4;
    case ATTN_DTYPE_I32: return 4;
    case ATTN_DTYPE_U8: return 1;
    case ATTN_DTYPE_I64: return 8;
    case ATTN_DTYPE_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool valid_dtype(int32_t dt) { return dt >= ATTN_DTYPE_BF16 && dt <= ATTN_DTYPE_FP8_E4M3; }

// A usable scale is finite and so is scale * log2(e), the factor the kernels
// apply in the exp2 domain (|scale| below about 2.36e38).
bool scale_ok(float scale) {
  const float s2 = scale * attn::kLog2e;
  return scale == scale && s2 - s2 == 0.0f;
}

// Rank, non-negative sizes / strides, unit inner stride.
// A NULL data pointer is accepted only for an empty tensor.
int check_tensor(const attn_tensor* t, int ndim) {
  if (!t) return ATTN_ERR_NULL;
  if (!valid_dtype(t->dtype)) return ATTN_ERR_ENUM;
  if (t->ndim != ndim) return ATTN_ERR_SHAPE;
  bool empty = false;
  for (int d = 0; d < ndim; ++d) {
    if (t->shape[d] < 0) return ATTN_ERR_SHAPE;
    if (t->stride[d] < 0) return ATTN_ERR_STRIDE;
    empty = empty || t->shape[d] == 0;
  }
  if (!t->data && !empty) return ATTN_ERR_NULL;
  if (t->stride[ndim - 1] != 1) return ATTN_ERR_STRIDE;
  return ATTN_OK;
}

// Rows of [rows, heads, dim] tensors must start on 16-byte boundaries, must
// not overlap (a row stride of at least the head dim), and one 64-row tile of
// them must span less than 2^31 bytes (kernels address tiles with 32-bit
// byte offsets).
int check_rows_aligned(const attn_tensor* t) {
  const int es = elem_size(t->dtype);
  const int64_t per16 = 16 / es;
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0) return ATTN_ERR_STRIDE;
  if (t->stride[0] % per16 != 0 || t->stride[1] % per16 != 0) return ATTN_ERR_STRIDE;
  if (t->shape[0] > 1 && t->stride[0] < t->shape[2]) return ATTN_ERR_STRIDE;
  if (t->stride[0] * es * 64 >= ((int64_t)1 << 31)) return ATTN_ERR_RANGE;
  return ATTN_OK;
}

int prepare(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t mask_kind,
            const attn_mask_arg* mask, const float* sinks, int32_t sink_mode, float scale,
            const attn_tensor* out, const float* lse, Params* P, Instance* inst) {
  *inst = kInstNone;
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (mask_kind < ATTN_MASK_WINDOW || mask_kind > ATTN_MASK_BLOCKSEL) return ATTN_ERR_ENUM;
  if (sink_mode < ATTN_SINK_NONE || sink_mode > ATTN_SINK_NULL_LOGIT) return ATTN_ERR_ENUM;
  if (!mask) return ATTN_ERR_NULL;
  int rc;
  if ((rc = check_tensor(q, 3)) || (rc = check_tensor(k, 3)) || (rc = check_tensor(v, 3)) ||
      (rc = check_tensor(out, 3)))
    return rc;
  const int32_t dt = q->dtype;
  if (dt != ATTN_DTYPE_BF16 && dt != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (k->dtype != dt || v->dtype != dt || out->dtype != dt) return ATTN_ERR_DTYPE;

  const int64_t T = q->shape[0], Hq = q->shape[1], Dqk = q->shape[2];
  const int64_t Tk = k->shape[0], Hkv = k->shape[1], Dv = v->shape[2];
  if (k->shape[2] != Dqk || v->shape[0] != Tk || v->shape[1] != Hkv) return ATTN_ERR_SHAPE;
  if (out->shape[0] != T || out->shape[1] != Hq || out->shape[2] != Dv) return ATTN_ERR_SHAPE;
  if (Hq < 1 || Hkv < 1 || Dqk < 1 || Dv < 1) return ATTN_ERR_SHAPE;
  if (T > kMaxTokens || Tk > kMaxTokens || Hq > 65535 || Hq * T > (int64_t)0x7fffffff * 4)
    return ATTN_ERR_RANGE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if ((rc = check_rows_aligned(q)) || (rc = check_rows_aligned(k)) || (rc = check_rows_aligned(v)) ||
      (rc = check_rows_aligned(out)))
    return rc;
  if (!lse && T > 0) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_STRIDE;
  if (sink_mode != ATTN_SINK_NONE && !sinks) return ATTN_ERR_NULL;
  if (!scale_ok(scale)) return ATTN_ERR_RANGE;

  memset(P, 0, sizeof(*P));
  P->q = q->data; P->k = k->data; P->v = v->data; P->out = out->data;
  P->lse = const_cast<float*>(lse);
  P->cu = cu_seqlens;
  P->sinks = sinks;
  P->q_row = q->stride[0]; P->q_head = q->stride[1];
  P->k_row = k->stride[0]; P->k_head = k->stride[1];
  P->v_row = v->stride[0]; P->v_head = v->stride[1];
  P->o_row = out->stride[0]; P->o_head = out->stride[1];
  P->T = (int)T; P->Tk = (int)Tk; P->Hq = (int)Hq; P->Hkv = (int)Hkv; P->group = (int)(Hq / Hkv);
  P->Dqk = (int)Dqk; P->Dv = (int)Dv;
  P->num_seqs = num_seqs;
  P->scale_log2 = scale * attn::kLog2e;

  if (mask_kind == ATTN_MASK_WINDOW || mask_kind == ATTN_MASK_BLOCKSEL) {
    if (T != Tk) return ATTN_ERR_SHAPE;
    if (T > 0 && (!cu_seqlens || num_seqs < 1)) return cu_seqlens ? ATTN_ERR_RANGE : ATTN_ERR_NULL;
  }
  if (mask_kind == ATTN_MASK_WINDOW) {
    if (mask->window < 0) return ATTN_ERR_RANGE;
    // a window of T or more keys covers every sequence whole: clamp, so that
    // no row +- window sum can leave the int32 range
    P->window = (int)(mask->window < T ? mask->window : T);
  } else if (mask_kind == ATTN_MASK_TOPK) {
    const attn_tensor* ti = mask->topk_idx;
    if ((rc = check_tensor(ti, 2))) return rc;
    if (ti->dtype != ATTN_DTYPE_I32) return ATTN_ERR_DTYPE;
    if (ti->shape[0] != T) return ATTN_ERR_SHAPE;
    if (ti->shape[1] > kMaxTokens) return ATTN_ERR_RANGE;
    if (reinterpret_cast<uintptr_t>(ti->data) % 4 != 0) return ATTN_ERR_STRIDE;
    P->topk_idx = static_cast<const int32_t*>(ti->data);
    P->topk_row = ti->stride[0];
    P->topk = (int)ti->shape[1];
    if (sink_mode == ATTN_SINK_KEY0_BIAS) return ATTN_ERR_UNSUPPORTED;
  } else {
    const attn_tensor* bs = mask->block_sel;
    if ((rc = check_tensor(bs, 4))) return rc;
    if (bs->dtype != ATTN_DTYPE_U8) return ATTN_ERR_DTYPE;
    if (mask->block_size < 1) return ATTN_ERR_RANGE;
    if (bs->shape[0] != 1 || bs->shape[2] != T) return ATTN_ERR_SHAPE;
    const int64_t Hidx = bs->shape[1], NB = bs->shape[3];
    if (Hidx < 1 || Hq % Hidx != 0) return ATTN_ERR_HEADS;
    if (NB < (T + mask->block_size - 1) / mask->block_size || NB > kMaxTokens) return ATTN_ERR_SHAPE;
    P->bsel = static_cast<const uint8_t*>(bs->data);
    P->bsel_head = bs->stride[1];
    P->bsel_q = bs->stride[2];
    P->Hidx = (int)Hidx;
    P->NB = (int)NB;
    P->block_size = mask->block_size;
  }

  // kernel instance, then its grid against the launch limit
  int64_t items = 0;
  if (dt == ATTN_DTYPE_F32) {
    if (Dqk > 576 || Dv > 576) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstGenericF32;
    items = attn::generic_f32_items(*P);
  } else if (mask_kind == ATTN_MASK_WINDOW) {
    if (Dqk != Dv || !(Dqk == 64 || Dqk == 80 || Dqk == 96 || Dqk == 128)) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstWindowBf16;
    items = attn::window_bf16_items(*P);
  } else if (mask_kind == ATTN_MASK_TOPK) {
    const bool shared_latent = v->data == k->data && v->stride[0] == k->stride[0] && Hkv == 1;
    if (!shared_latent || Dqk != 576 || Dv != 512 || Hq % 64 != 0) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstTopkMlaBf16;
    items = attn::topk_mla_bf16_items(*P);
  } else {
    if (Dqk != 128 || Dv != 128 || Hq / Hkv != 4 || mask->block_size != 64 || Hkv % P->Hidx != 0)
      return ATTN_ERR_UNSUPPORTED;
    *inst = kInstBlockselBf16;
    items = attn::blocksel_bf16_items(*P);
  }
  if (items > kMaxGridItems) {
    *inst = kInstNone;
    return ATTN_ERR_RANGE;
  }
  return ATTN_OK;
}

}  // namespace

ATTN_API int attn_sink_check(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t mask_kind,
                             const attn_mask_arg* mask, const float* sinks, int32_t sink_mode,
                             float scale, const attn_tensor* out, const float* lse) {
  Params P;
  Instance inst;
  return prepare(q, k, v, cu_seqlens, num_seqs, mask_kind, mask, sinks, sink_mode, scale, out, lse,
                 &P, &inst);
}

ATTN_API int attn_sink_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, int32_t mask_kind,
                           const attn_mask_arg* mask, const float* sinks, int32_t sink_mode,
                           float scale, const attn_tensor* out, float* lse, hipStream_t stream) {
  Params P;
  Instance inst;
  int rc = prepare(q, k, v, cu_seqlens, num_seqs, mask_kind, mask, sinks, sink_mode, scale, out, lse,
                   &P, &inst);
  if (rc != ATTN_OK) return rc;
  if (P.T == 0) return ATTN_OK;
  hipError_t e = hipSuccess;
  switch (inst) {
    case kInstGenericF32: e = attn::launch_generic_f32(P, mask_kind, sink_mode, stream); break;
    case kInstWindowBf16: e = attn::launch_window_bf16(P, sink_mode, stream); break;
    case kInstTopkMlaBf16: e = attn::launch_topk_mla_bf16(P, sink_mode, stream); break;
    case kInstBlockselBf16: e = attn::launch_blocksel_bf16(P, sink_mode, stream); break;
    default: return ATTN_ERR_UNSUPPORTED;
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

namespace {

// ---------------------------------------------------------------- key-0 correction
int prepare_key0(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t window, const float* sinks,
                 float scale, const attn_tensor* out, const float* lse, attn::Key0Params* P,
                 bool* f32) {
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  int rc;
  if ((rc = check_tensor(q, 3)) || (rc = check_tensor(k, 3)) || (rc = check_tensor(v, 3)) ||
      (rc = check_tensor(out, 3)))
    return rc;
  const int32_t dt = q->dtype;
  if (dt != ATTN_DTYPE_BF16 && dt != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  if (k->dtype != dt || v->dtype != dt || out->dtype != dt) return ATTN_ERR_DTYPE;
  const int64_t T = q->shape[0], Hq = q->shape[1], Dqk = q->shape[2];
  const int64_t Hkv = k->shape[1], Dv = v->shape[2];
  if (k->shape[0] != T || v->shape[0] != T || out->shape[0] != T) return ATTN_ERR_SHAPE;
  if (k->shape[2] != Dqk || v->shape[1] != Hkv || out->shape[1] != Hq || out->shape[2] != Dv)
    return ATTN_ERR_SHAPE;
  if (Hq < 1 || Hkv < 1 || Dqk < 1 || Dv < 1) return ATTN_ERR_SHAPE;
  if (T > kMaxTokens || Hq > 4 * 65535) return ATTN_ERR_RANGE;
  if (Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if ((rc = check_rows_aligned(q)) || (rc = check_rows_aligned(k)) || (rc = check_rows_aligned(v)) ||
      (rc = check_rows_aligned(out)))
    return rc;
  const int per16 = 16 / elem_size(dt);
  if (Dqk % per16 != 0 || Dv % per16 != 0) return ATTN_ERR_UNSUPPORTED;
  if (!lse && T > 0) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_STRIDE;
  if (!sinks) return ATTN_ERR_NULL;
  if (T > 0 && (!cu_seqlens || num_seqs < 1)) return cu_seqlens ? ATTN_ERR_RANGE : ATTN_ERR_NULL;
  if (window < 0) return ATTN_ERR_RANGE;
  if (window > T) window = (int32_t)T;  // rows past T do not exist: same affected rows
  // one 256-lane workgroup per (row slot, group of 4 heads)
  if ((int64_t)num_seqs * ((int64_t)window + 1) * 256 > kMaxGridItems) return ATTN_ERR_RANGE;
  if (!scale_ok(scale)) return ATTN_ERR_RANGE;
  memset(P, 0, sizeof(*P));
  P->q = q->data; P->k = k->data; P->v = v->data; P->out = out->data;
  P->lse = const_cast<float*>(lse);
  P->cu = cu_seqlens; P->sinks = sinks;
  P->q_row = q->stride[0]; P->q_head = q->stride[1];
  P->k_row = k->stride[0]; P->k_head = k->stride[1];
  P->v_row = v->stride[0]; P->v_head = v->stride[1];
  P->o_row = out->stride[0]; P->o_head = out->stride[1];
  P->T = (int)T; P->Hq = (int)Hq; P->group = (int)(Hq / Hkv); P->Dqk = (int)Dqk; P->Dv = (int)Dv;
  P->num_seqs = num_seqs; P->window = window; P->scale = scale;
  *f32 = dt == ATTN_DTYPE_F32;
  return ATTN_OK;
}

// ---------------------------------------------------------------- merge
int prepare_merge(const attn_tensor* parts_out, const float* const* parts_lse, int32_t num_parts,
                  const float* sinks, int32_t sink_mode, const attn_tensor* out, const float* lse,
                  attn::MergeParams* P, bool* f32) {
  if (!parts_out || !parts_lse || !out) return ATTN_ERR_NULL;
  if (num_parts < 1 || num_parts > attn::kMergeMaxParts) return ATTN_ERR_RANGE;
  if (sink_mode < ATTN_SINK_NONE || sink_mode > ATTN_SINK_NULL_LOGIT) return ATTN_ERR_ENUM;
  if (sink_mode == ATTN_SINK_KEY0_BIAS) return ATTN_ERR_UNSUPPORTED;
  if (sink_mode == ATTN_SINK_NULL_LOGIT && !sinks) return ATTN_ERR_NULL;
  int rc;
  if ((rc = check_tensor(out, 3))) return rc;
  const int32_t dt = out->dtype;
  if (dt != ATTN_DTYPE_BF16 && dt != ATTN_DTYPE_F32) return ATTN_ERR_DTYPE;
  const int64_t T = out->shape[0], Hq = out->shape[1], Dv = out->shape[2];
  if (Hq < 1 || Dv < 1) return ATTN_ERR_SHAPE;
  if (T > kMaxTokens || Hq > 65535) return ATTN_ERR_RANGE;
  if ((rc = check_rows_aligned(out))) return rc;
  if (Dv % (16 / elem_size(dt)) != 0) return ATTN_ERR_UNSUPPORTED;
  if (!lse && T > 0) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_STRIDE;
  memset(P, 0, sizeof(*P));
  for (int p = 0; p < num_parts; ++p) {
    const attn_tensor* t = parts_out + p;
    if ((rc = check_tensor(t, 3))) return rc;
    if (t->dtype != dt) return ATTN_ERR_DTYPE;
    if (t->shape[0] != T || t->shape[1] != Hq || t->shape[2] != Dv) return ATTN_ERR_SHAPE;
    if ((rc = check_rows_aligned(t))) return rc;
    if (!parts_lse[p] && T > 0) return ATTN_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(parts_lse[p]) % 4 != 0) return ATTN_ERR_STRIDE;
    if (T > 0 && (t->data == out->data || parts_lse[p] == lse)) return ATTN_ERR_RANGE;  // no in-place merge
    P->part_out[p] = t->data;
    P->part_lse[p] = parts_lse[p];
    P->p_row[p] = t->stride[0];
    P->p_head[p] = t->stride[1];
  }
  P->out = out->data;
  P->lse = const_cast<float*>(lse);
  P->sinks = sinks;
  P->o_row = out->stride[0]; P->o_head = out->stride[1];
  P->T = (int)T; P->Hq = (int)Hq; P->Dv = (int)Dv; P->nparts = num_parts;
  P->nchunks = T * Hq * (Dv / (16 / elem_size(dt)));
  *f32 = dt == ATTN_DTYPE_F32;
  return ATTN_OK;
}

}  // namespace

ATTN_API int attn_sink_key0_correct_check(const attn_tensor* q, const attn_tensor* k,
                                          const attn_tensor* v, const int32_t* cu_seqlens,
                                          int32_t num_seqs, int32_t window, const float* sinks,
                                          float scale, const attn_tensor* out, const float* lse) {
  attn::Key0Params P;
  bool f32;
  return prepare_key0(q, k, v, cu_seqlens, num_seqs, window, sinks, scale, out, lse, &P, &f32);
}

ATTN_API int attn_sink_key0_correct(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                    const int32_t* cu_seqlens, int32_t num_seqs, int32_t window,
                                    const float* sinks, float scale, const attn_tensor* out, float* lse,
                                    hipStream_t stream) {
  attn::Key0Params P;
  bool f32;
  const int rc = prepare_key0(q, k, v, cu_seqlens, num_seqs, window, sinks, scale, out, lse, &P, &f32);
  if (rc != ATTN_OK) return rc;
  if (P.T == 0) return ATTN_OK;
  return attn::launch_key0_correct(P, f32, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_API int attn_sink_merge_check(const attn_tensor* parts_out, const float* const* parts_lse,
                                   int32_t num_parts, const float* sinks, int32_t sink_mode,
                                   const attn_tensor* out, const float* lse) {
  attn::MergeParams P;
  bool f32;
  return prepare_merge(parts_out, parts_lse, num_parts, sinks, sink_mode, out, lse, &P, &f32);
}

ATTN_API int attn_sink_merge(const attn_tensor* parts_out, const float* const* parts_lse,
                             int32_t num_parts, const float* sinks, int32_t sink_mode,
                             const attn_tensor* out, float* lse, hipStream_t stream) {
  attn::MergeParams P;
  bool f32;
  const int rc = prepare_merge(parts_out, parts_lse, num_parts, sinks, sink_mode, out, lse, &P, &f32);
  if (rc != ATTN_OK) return rc;
  if (P.T == 0) return ATTN_OK;
  return attn::launch_merge(P, f32, sink_mode == ATTN_SINK_NULL_LOGIT, stream) == hipSuccess
             ? ATTN_OK : ATTN_ERR_LAUNCH;
}

namespace {

// ---------------------------------------------------------------- context-parallel reorder
int prepare_cp_slots(int32_t cp_size, int64_t t_local, int32_t rank, const int64_t* slots,
                     attn::CpSlotsParams* P) {
  if (cp_size < 1 || t_local < 0 || t_local % 2 != 0 || t_local > ((int64_t)1 << 40)) return ATTN_ERR_RANGE;
  if (rank < -1 || rank >= cp_size) return ATTN_ERR_RANGE;
  const int64_t n = rank < 0 ? (int64_t)cp_size * t_local : t_local;
  if (n > 0 && !slots) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(slots) % 8 != 0) return ATTN_ERR_STRIDE;
  P->slots = const_cast<int64_t*>(slots);
  P->t_local = t_local;
  P->n = n;
  P->cp_size = cp_size;
  P->rank = rank;
  return ATTN_OK;
}

// Rank 1..4 tensors whose rows (everything past dim 0) are dense.
int check_rows_tensor(const attn_tensor* t, int64_t* row_bytes) {
  if (!t) return ATTN_ERR_NULL;
  if (!valid_dtype(t->dtype)) return ATTN_ERR_ENUM;
  if (t->ndim < 1 || t->ndim > 4) return ATTN_ERR_SHAPE;
  int64_t dense = 1;
  bool empty = false;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] < 0) return ATTN_ERR_SHAPE;
    if (t->stride[d] < 0) return ATTN_ERR_STRIDE;
    empty = empty || t->shape[d] == 0;
    if (d > 0) {
      if (t->stride[d] != dense && t->shape[d] > 1) return ATTN_ERR_STRIDE;
      dense *= t->shape[d];
    }
  }
  if (!t->data && !empty) return ATTN_ERR_NULL;
  *row_bytes = dense * elem_size(t->dtype);
  if (t->shape[0] > 1 && t->stride[0] < dense) return ATTN_ERR_STRIDE;
  return ATTN_OK;
}

// Widest chunk (16, 8 or 4 bytes) dividing the row length, both row strides
// and both base addresses; 0 if not even 4 does.
int chunk_width(int64_t row_bytes, const attn_tensor* a, const attn_tensor* b) {
  const uint64_t bits = (uint64_t)row_bytes | (uint64_t)(a->stride[0] * elem_size(a->dtype)) |
                        (uint64_t)(b->stride[0] * elem_size(b->dtype)) |
                        (uint64_t)reinterpret_cast<uintptr_t>(a->data) | (uint64_t)reinterpret_cast<uintptr_t>(b->data);
  return bits % 16 == 0 ? 16 : bits % 8 == 0 ? 8 : bits % 4 == 0 ? 4 : 0;
}

int prepare_permute(const attn_tensor* src, const int64_t* index, int64_t n, int32_t scatter,
                    const attn_tensor* dst, attn::PermuteParams* P) {
  if (!src || !dst) return ATTN_ERR_NULL;
  if (scatter != 0 && scatter != 1) return ATTN_ERR_ENUM;
  int64_t rs, rd;
  int rc;
  if ((rc = check_rows_tensor(src, &rs)) || (rc = check_rows_tensor(dst, &rd))) return rc;
  if (src->dtype != dst->dtype) return ATTN_ERR_DTYPE;
  if (src->ndim != dst->ndim) return ATTN_ERR_SHAPE;
  for (int d = 1; d < src->ndim; ++d)
    if (src->shape[d] != dst->shape[d]) return ATTN_ERR_SHAPE;
  if (n < 0 || (scatter ? src->shape[0] : dst->shape[0]) != n) return ATTN_ERR_SHAPE;
  const int cw = chunk_width(rs, src, dst);
  if (cw == 0 || rs / cw > 0x7fffffff) return ATTN_ERR_UNSUPPORTED;
  if (n > 0 && !index) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(index) % 8 != 0) return ATTN_ERR_STRIDE;
  if (n > 0 && rs > 0 && src->data == dst->data) return ATTN_ERR_RANGE;  // not in place
  const int es = elem_size(src->dtype);
  P->src = static_cast<const char*>(src->data);
  P->dst = static_cast<char*>(dst->data);
  P->index = index;
  P->src_row = src->stride[0] * es;
  P->dst_row = dst->stride[0] * es;
  P->src_rows = src->shape[0];
  P->dst_rows = dst->shape[0];
  P->n = n;
  P->chunks = (int)(rs / cw);
  P->chunk_bytes = cw;
  P->scatter = scatter;
  return ATTN_OK;
}

int prepare_cp_documents(const int64_t* positions, int64_t T, const int32_t* doc_ids, const int32_t* cu_seqlens,
                         int32_t max_docs, const int32_t* num_docs, attn::CpDocParams* P) {
  if (T < 0 || T > kMaxTokens || max_docs < 0) return ATTN_ERR_RANGE;
  if (T > 0 && !positions) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(positions) % 8 != 0 || reinterpret_cast<uintptr_t>(doc_ids) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(cu_seqlens) % 4 != 0 || reinterpret_cast<uintptr_t>(num_docs) % 4 != 0)
    return ATTN_ERR_STRIDE;
  P->positions = positions;
  P->T = T;
  P->doc_ids = const_cast<int32_t*>(doc_ids);
  P->cu = const_cast<int32_t*>(cu_seqlens);
  P->num_docs = const_cast<int32_t*>(num_docs);
  P->max_docs = max_docs;
  return ATTN_OK;
}

}  // namespace

ATTN_API int attn_sink_cp_slots_check(int32_t cp_size, int64_t t_local, int32_t rank, const int64_t* slots) {
  attn::CpSlotsParams P;
  return prepare_cp_slots(cp_size, t_local, rank, slots, &P);
}

ATTN_API int attn_sink_cp_slots(int32_t cp_size, int64_t t_local, int32_t rank, int64_t* slots,
                                hipStream_t stream) {
  attn::CpSlotsParams P;
  const int rc = prepare_cp_slots(cp_size, t_local, rank, slots, &P);
  if (rc != ATTN_OK || P.n == 0) return rc;
  return attn::launch_cp_slots(P, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_API int attn_sink_cp_permute_rows_check(const attn_tensor* src, const int64_t* index, int64_t n,
                                             int32_t scatter, const attn_tensor* dst) {
  attn::PermuteParams P;
  return prepare_permute(src, index, n, scatter, dst, &P);
}

ATTN_API int attn_sink_cp_permute_rows(const attn_tensor* src, const int64_t* index, int64_t n, int32_t scatter,
                                       const attn_tensor* dst, hipStream_t stream) {
  attn::PermuteParams P;
  const int rc = prepare_permute(src, index, n, scatter, dst, &P);
  if (rc != ATTN_OK || P.n == 0 || P.chunks == 0) return rc;
  return attn::launch_permute_rows(P, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_API int attn_sink_cp_documents_check(const int64_t* positions, int64_t T, const int32_t* doc_ids,
                                          const int32_t* cu_seqlens, int32_t max_docs, const int32_t* num_docs) {
  attn::CpDocParams P;
  return prepare_cp_documents(positions, T, doc_ids, cu_seqlens, max_docs, num_docs, &P);
}

ATTN_API int attn_sink_cp_documents(const int64_t* positions, int64_t T, int32_t* doc_ids, int32_t* cu_seqlens,
                                    int32_t max_docs, int32_t* num_docs, hipStream_t stream) {
  attn::CpDocParams P;
  const int rc = prepare_cp_documents(positions, T, doc_ids, cu_seqlens, max_docs, num_docs, &P);
  if (rc != ATTN_OK) return rc;
  if (!doc_ids && !cu_seqlens && !num_docs) return ATTN_OK;
  return attn::launch_cp_documents(P, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

namespace {

// ---------------------------------------------------------------- fp8 sparse-MLA decode
int64_t decode_ws_bytes(int64_t T, int64_t Hq, int nsplit) {
  return (int64_t)nsplit * T * Hq * (512 * 4 + 4);
}

int prepare_decode(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale, const attn_tensor* ti,
                   const float* sinks, int32_t sink_mode, float scale, const attn_tensor* out, const float* lse,
                   const void* ws, int64_t ws_bytes, attn::DecodeParams* P) {
  if (!q || !kv || !ti || !out) return ATTN_ERR_NULL;
  if (sink_mode < ATTN_SINK_NONE || sink_mode > ATTN_SINK_NULL_LOGIT) return ATTN_ERR_ENUM;
  if (sink_mode == ATTN_SINK_KEY0_BIAS) return ATTN_ERR_UNSUPPORTED;
  if (sink_mode == ATTN_SINK_NULL_LOGIT && !sinks) return ATTN_ERR_NULL;
  int rc;
  if ((rc = check_tensor(q, 3)) || (rc = check_tensor(kv, 3)) || (rc = check_tensor(out, 3)) ||
      (rc = check_tensor(ti, 2)))
    return rc;
  if (q->dtype != ATTN_DTYPE_BF16 || out->dtype != ATTN_DTYPE_BF16 || kv->dtype != ATTN_DTYPE_FP8_E4M3 ||
      ti->dtype != ATTN_DTYPE_I32)
    return ATTN_ERR_DTYPE;
  const int64_t T = q->shape[0], Hq = q->shape[1], Tk = kv->shape[0];
  if (q->shape[2] != 576 || kv->shape[1] != 1 || kv->shape[2] != 576 || out->shape[2] != 512)
    return ATTN_ERR_UNSUPPORTED;
  if (out->shape[0] != T || out->shape[1] != Hq || ti->shape[0] != T) return ATTN_ERR_SHAPE;
  if (Hq < 64 || Hq % 64 != 0) return ATTN_ERR_UNSUPPORTED;
  if (T > kMaxTokens || Tk > kMaxTokens || ti->shape[1] > kMaxTokens || Hq > 65535) return ATTN_ERR_RANGE;
  if ((rc = check_rows_aligned(q)) || (rc = check_rows_aligned(out))) return rc;
  if (reinterpret_cast<uintptr_t>(kv->data) % 16 != 0 || kv->stride[0] % 16 != 0) return ATTN_ERR_STRIDE;
  if (Tk > 1 && kv->stride[0] < 576) return ATTN_ERR_STRIDE;
  if (Tk > 0 && !kv_scale) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(kv_scale) % 4 != 0 || reinterpret_cast<uintptr_t>(ti->data) % 4 != 0)
    return ATTN_ERR_STRIDE;
  if (!lse && T > 0) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return ATTN_ERR_STRIDE;
  if (!scale_ok(scale)) return ATTN_ERR_RANGE;
  if (T * (Hq / 64) * 256 > kMaxGridItems) return ATTN_ERR_RANGE;  // one 256-lane workgroup per (row, 64 heads, piece)
  const int nsplit = attn::decode_splits(T, Hq, ti->shape[1]);
  if (T > 0 && (!ws || ws_bytes < decode_ws_bytes(T, Hq, nsplit))) return ws ? ATTN_ERR_RANGE : ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(ws) % 16 != 0) return ATTN_ERR_STRIDE;
  memset(P, 0, sizeof(*P));
  P->q = q->data; P->k = kv->data; P->kv_scale = kv_scale; P->topk_idx = static_cast<const int32_t*>(ti->data);
  P->sinks = sinks; P->out = out->data; P->lse = const_cast<float*>(lse);
  P->ws_out = static_cast<float*>(const_cast<void*>(ws));
  P->ws_lse = P->ws_out + (int64_t)nsplit * T * Hq * 512;
  P->q_row = q->stride[0]; P->q_head = q->stride[1]; P->k_row = kv->stride[0];
  P->o_row = out->stride[0]; P->o_head = out->stride[1]; P->topk_row = ti->stride[0];
  P->T = (int)T; P->Tk = (int)Tk; P->Hq = (int)Hq; P->topk = (int)ti->shape[1];
  P->nsplit = nsplit; P->split_len = attn::decode_split_len(ti->shape[1], nsplit);
  P->scale_log2 = scale * attn::kLog2e;
  return ATTN_OK;
}

}  // namespace

ATTN_API int attn_sink_mla_decode_fp8_workspace(int64_t T, int64_t Hq, int64_t topk, int64_t* bytes) {
  if (!bytes) return ATTN_ERR_NULL;
  if (T < 0 || Hq < 64 || Hq % 64 != 0 || topk < 0 || T > kMaxTokens || topk > kMaxTokens) return ATTN_ERR_RANGE;
  *bytes = decode_ws_bytes(T, Hq, attn::decode_splits(T, Hq, topk));
  return ATTN_OK;
}

ATTN_API int attn_sink_mla_decode_fp8_check(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                                            const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode,
                                            float scale, const attn_tensor* out, const float* lse,
                                            const void* workspace, int64_t workspace_bytes) {
  attn::DecodeParams P;
  return prepare_decode(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse, workspace, workspace_bytes, &P);
}

ATTN_API int attn_sink_mla_decode_fp8(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                                      const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode,
                                      float scale, const attn_tensor* out, float* lse, void* workspace,
                                      int64_t workspace_bytes, hipStream_t stream) {
  attn::DecodeParams P;
  const int rc = prepare_decode(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse, workspace,
                                workspace_bytes, &P);
  if (rc != ATTN_OK || P.T == 0) return rc;
  return attn::launch_mla_decode_fp8(P, sink_mode, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_API int attn_sink_mla_decode_fp8_noalloc(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                                              const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode,
                                              float scale, const attn_tensor* out, float* lse, hipStream_t stream) {
  static_assert(attn::kDecodeScratchBytes == ATTN_SINK_DECODE_SCRATCH_BYTES, "scratch limit");
  attn::DecodeParams P;
  // validate against the scratch limit first (a placeholder address: no
  // device access), so a refused call makes no HIP call at all
  int rc = prepare_decode(q, kv, kv_scale, topk_idx, sinks, sink_mode, scale, out, lse,
                          reinterpret_cast<const void*>((uintptr_t)256), attn::kDecodeScratchBytes, &P);
  if (rc != ATTN_OK || P.T == 0) return rc;
  void* base = nullptr;
  if (attn::decode_scratch_address(&base) != hipSuccess) return ATTN_ERR_LAUNCH;
  P.ws_out = static_cast<float*>(base);
  P.ws_lse = P.ws_out + (int64_t)P.nsplit * P.T * P.Hq * 512;
  return attn::launch_mla_decode_fp8(P, sink_mode, stream) == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

ATTN_API const char* attn_sink_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_ENUM: return "mask_kind, sink_mode or a dtype is out of range";
    case ATTN_ERR_SHAPE: return "tensor ranks or sizes disagree";
    case ATTN_ERR_STRIDE: return "non-unit inner stride or a row not 16-byte aligned";
    case ATTN_ERR_HEADS: return "head counts do not divide (Hq % Hkv or Hq % Hidx)";
    case ATTN_ERR_DTYPE: return "dtype not allowed for this argument";
    case ATTN_ERR_UNSUPPORTED: return "no kernel instance covers this combination";
    case ATTN_ERR_RANGE: return "a size or value is out of range";
    case ATTN_ERR_LAUNCH: return "the kernel launch failed";
    default: return "unknown status";
  }
}

ATTN_API int attn_sink_abi_version(void) { return ATTN_SINK_ABI_VERSION; }
