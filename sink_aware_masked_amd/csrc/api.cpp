// C ABI front end: argument validation, kernel-instance selection and a single
// launch on the caller's stream.  No allocation, no synchronisation, no device
// reads from the host.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "attn_sink.h"
#include "common.hpp"
#include "compose.hpp"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace attn {
hipError_t launch_window_bf16(const Params& p, int sink, hipStream_t st);
hipError_t launch_generic_f32(const Params& p, int mask, int sink, hipStream_t st);
hipError_t launch_topk_mla_bf16(const Params& p, int sink, hipStream_t st);
hipError_t launch_blocksel_bf16(const Params& p, int sink, hipStream_t st);
}  // namespace attn

static_assert(attn::kMergeMaxParts == ATTN_SINK_MERGE_MAX_PARTS, "merge part limit");

namespace {

using attn::Params;

enum Instance { kInstNone = 0, kInstGenericF32, kInstWindowBf16, kInstTopkMlaBf16, kInstBlockselBf16 };

constexpr int64_t kMaxTokens = 0x7fffffffLL;

int elem_size(int32_t dt) {
  switch (dt) {
    case ATTN_DTYPE_BF16: return 2;
    case ATTN_DTYPE_F32: return 4;
    case ATTN_DTYPE_I32: return 4;
    case ATTN_DTYPE_U8: return 1;
    default: return 0;
  }
}

bool valid_dtype(int32_t dt) { return dt >= ATTN_DTYPE_BF16 && dt <= ATTN_DTYPE_U8; }

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
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return ATTN_ERR_RANGE;

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
    P->window = mask->window;
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

  // kernel instance
  if (dt == ATTN_DTYPE_F32) {
    if (Dqk > 576 || Dv > 576) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstGenericF32;
    return ATTN_OK;
  }
  if (mask_kind == ATTN_MASK_WINDOW) {
    if (Dqk != Dv || !(Dqk == 64 || Dqk == 80 || Dqk == 96 || Dqk == 128)) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstWindowBf16;
    return ATTN_OK;
  }
  if (mask_kind == ATTN_MASK_TOPK) {
    const bool shared_latent = v->data == k->data && v->stride[0] == k->stride[0] && Hkv == 1;
    if (!shared_latent || Dqk != 576 || Dv != 512 || Hq % 64 != 0) return ATTN_ERR_UNSUPPORTED;
    *inst = kInstTopkMlaBf16;
    return ATTN_OK;
  }
  if (Dqk != 128 || Dv != 128 || Hq / Hkv != 4 || mask->block_size != 64 || Hkv % P->Hidx != 0)
    return ATTN_ERR_UNSUPPORTED;
  *inst = kInstBlockselBf16;
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
  if ((int64_t)num_seqs * ((int64_t)window + 1) > kMaxTokens) return ATTN_ERR_RANGE;
  if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
    return ATTN_ERR_RANGE;
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
