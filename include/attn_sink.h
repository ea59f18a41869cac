/*
 * attn_sink.h -- C ABI of the sink-aware masked attention forward library
 * (gfx950 / MI355X).
 *
 * attn_sink_fwd computes, for every packed query row i and query head h,
 *
 *     out[i, h, :] = softmax over the key set S(i, h) (plus the sink) of
 *                    scale * q[i, h, :] . k[j, h / (Hq/Hkv), :]   applied to v
 *     lse[h, i]    = natural-log log-sum-exp of those scaled logits over the
 *                    selected keys (never over the null-logit sink)
 *
 * Two more entry points act on such (out, lse) pairs: attn_sink_merge
 * combines results over disjoint key sets and folds the sink in after the
 * merge, and attn_sink_key0_correct applies the key-0 sink to a finished
 * no-sink window result in closed form (the unfused design, kept as a
 * comparator for the fused one).  The attn_sink_cp_* calls are the
 * context-parallel reorder primitives that bring sharded K/V into global token
 * order and derive the document segments.
 *
 * Sources (page titles; sections / paragraphs named):
 *   - "[Bugfix][MiMo] Apply vision attention sinks in the window attention
 *     path" (vLLM): the symmetric window over cu_seqlens-packed sequences,
 *     the key0_bias sink (sinks[h] added to the logit of each sequence's first
 *     key), and the varlen LSE contract of shape (nheads, total_q).
 *   - "Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA Triton kernel":
 *     per-row top-k key lists with -1 padding over one shared latent KV, and
 *     the null_logit sink folded in after the key loop (Implementation
 *     paragraph): it joins only the softmax denominator, the LSE stays over
 *     the selected keys, and a sink of -inf leaves the result unchanged.
 *   - NeMo AutoModel "cp_sparse_attn" API page: a per-query block-selection
 *     table [B, index_heads, S, key_blocks] combined with token-causal and
 *     same-document masks (_flex_sparse_attention, _local_sparse_forward),
 *     fully masked rows giving zero output, and 64-bit table offsets
 *     (_block_sel_flat_offset).
 *
 * Conventions shared by all entry points
 *   - All tensor data pointers are DEVICE pointers; descriptors themselves
 *     live in host memory and are read during the call only.
 *   - Strides are in elements.  The innermost dimension of q, k, v and out must
 *     be contiguous (stride 1); the other strides are free but must keep every
 *     row 16-byte aligned (bf16: multiples of 8 elements; f32: of 4), and 64
 *     rows must span less than 2^31 bytes (kernels address inside a 64-row
 *     tile with 32-bit offsets from a 64-bit tile base; ATTN_ERR_RANGE
 *     otherwise).  Offsets across the whole tensor are 64-bit.
 *   - The caller owns every buffer, including the one scratch buffer (the fp8
 *     decode's workspace).  The library allocates nothing and keeps no
 *     mutable global state: calls are reentrant and may run concurrently on
 *     different streams.  The one exception is the allocation-free decode
 *     (attn_sink_mla_decode_fp8_noalloc), whose scratch is a static device
 *     array shared by all its calls on a GPU.  Inputs are read only.
 *     attn_sink_fwd and attn_sink_merge fully write out and lse (rows with an
 *     empty key set get out = 0 and lse = -inf); attn_sink_key0_correct
 *     updates them in place.
 *   - Each call enqueues a single kernel launch on `stream` (the fp8 decode
 *     two); no call ever synchronises or reads device memory from the host.
 *   - Errors are returned as negative attn_status codes.  Every argument error
 *     is detected on the host BEFORE anything is enqueued.  Device-side data
 *     (cu_seqlens contents, indices) is not validated -- see the
 *     preconditions below.
 */
#ifndef ATTN_SINK_H
#define ATTN_SINK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_SINK_ABI_VERSION 2

/* Which key set S(i, h) each query row attends to. */
typedef enum attn_mask_kind {
  /* Key j is valid iff it lies in the same cu_seqlens segment as query i and
   * |i - j| <= window (inclusive; symmetric, not causal).  q and k share the
   * packed token index space (T == Tk).  MiMo window-attention page. */
  ATTN_MASK_WINDOW = 0,
  /* Key j = topk_idx[i, t] for every t with 0 <= topk_idx[i, t] < Tk; any
   * other entry (-1 by convention) is padding and may sit anywhere in the
   * row.  One list per row, shared by all heads.  cu_seqlens is ignored.
   * DeepSeek-V4 sparse-MLA page. */
  ATTN_MASK_TOPK = 1,
  /* Key j is valid iff block_sel[0, h / (Hq/Hidx), i, j / block_size] != 0,
   * j <= i (token causal) and j lies in the same cu_seqlens segment
   * (document) as i.  T == Tk.  "cp_sparse_attn" page. */
  ATTN_MASK_BLOCKSEL = 2
} attn_mask_kind;

/* How sinks[h] enters the softmax. */
typedef enum attn_sink_mode {
  ATTN_SINK_NONE = 0,       /* no sink; `sinks` may be NULL                        */
  /* sinks[h] is added (unscaled) to the scaled logit of the first key of each
   * cu_seqlens segment whenever that key is in S(i, h); the LSE includes the
   * biased logit.  Not defined for ATTN_MASK_TOPK (no segments). */
  ATTN_SINK_KEY0_BIAS = 1,
  /* out = sum_j e^{l_j} v_j / (e^{sinks[h]} + sum_j e^{l_j}); the LSE is over
   * the selected keys only; sinks[h] = -inf reproduces ATTN_SINK_NONE bit for
   * bit. */
  ATTN_SINK_NULL_LOGIT = 2
} attn_sink_mode;

typedef enum attn_dtype {
  ATTN_DTYPE_BF16 = 0,
  ATTN_DTYPE_F32 = 1,
  ATTN_DTYPE_I32 = 2,
  ATTN_DTYPE_U8 = 3,
  ATTN_DTYPE_I64 = 4,  /* position ids / slot indices (context-parallel reorder) */
  ATTN_DTYPE_FP8_E4M3 = 5  /* OCP fp8 e4m3 (bias 7, max 448, no inf); fp8 latent cache */
} attn_dtype;

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL                       */
  ATTN_ERR_ENUM = -2,        /* mask_kind, sink_mode or a dtype is out of range  */
  ATTN_ERR_SHAPE = -3,       /* ranks or sizes disagree                          */
  ATTN_ERR_STRIDE = -4,      /* non-unit inner stride or misaligned rows         */
  ATTN_ERR_HEADS = -5,       /* Hq % Hkv != 0, or Hq % Hidx != 0                 */
  ATTN_ERR_DTYPE = -6,       /* dtypes disagree or are not allowed for a role    */
  ATTN_ERR_UNSUPPORTED = -7, /* well-formed, but no kernel instance covers it    */
  ATTN_ERR_RANGE = -8,       /* a size, stride or value is out of range (T >= 2^31, W < 0, 64 rows >= 2^31 bytes) */
  ATTN_ERR_LAUNCH = -9       /* the kernel launch itself failed                  */
} attn_status;

/* A strided view of a device array (up to 4 dimensions). */
typedef struct attn_tensor {
  void* data;          /* device pointer                                 */
  int32_t dtype;       /* attn_dtype                                     */
  int32_t ndim;        /* number of used entries in shape / stride       */
  int64_t shape[4];
  int64_t stride[4];   /* in elements                                    */
} attn_tensor;

/* Mask parameters; only the fields of the chosen mask kind are read. */
typedef struct attn_mask_arg {
  int32_t window;                /* WINDOW: W >= 0                                   */
  int32_t block_size;            /* BLOCKSEL: key block size in tokens (> 0)         */
  const attn_tensor* topk_idx;   /* TOPK: int32 [T, topk], row stride free, inner 1 */
  const attn_tensor* block_sel;  /* BLOCKSEL: uint8 [1, Hidx, T, NB], NB >= ceil(T/block_size), inner 1 */
} attn_mask_arg;

/*
 * attn_sink_fwd -- forward pass; enqueues one kernel on `stream`.
 *
 *   q          [T, Hq, Dqk]   bf16 or f32
 *   k          [Tk, Hkv, Dqk] same dtype as q
 *   v          [Tk, Hkv, Dv]  same dtype as q; may alias k (shared latent KV:
 *                             v->data == k->data with the same row stride and
 *                             Dv <= Dqk reads the first Dv columns of k)
 *   cu_seqlens device int32 [num_seqs + 1]; required (non-NULL, num_seqs >= 1)
 *              for WINDOW and BLOCKSEL, ignored for TOPK.
 *   mask_kind  attn_mask_kind;  mask: its parameters (host struct)
 *   sinks      device f32 [Hq]; required unless sink_mode == ATTN_SINK_NONE
 *   sink_mode  attn_sink_mode
 *   scale      multiplies q.k before the sink is applied (e.g. 1/sqrt(Dqk));
 *              must be finite with scale * log2(e) finite (|scale| < ~2.36e38),
 *              else ATTN_ERR_RANGE
 *   out        [T, Hq, Dv]    same dtype as q; must not overlap any input
 *   lse        device f32, dense [Hq, T]; must not overlap any input
 *   stream     HIP stream the kernel is enqueued on (0 = null stream)
 *
 * Kernel instances (anything else returns ATTN_ERR_UNSUPPORTED):
 *   f32  : every mask kind and sink mode, Dqk <= 576, Dv <= 576 (one wave per
 *          (row, head); exact-arithmetic reference-grade instance).
 *   bf16 : WINDOW   Dqk == Dv in {64, 80, 96, 128}, any Hq/Hkv grouping;
 *          TOPK     shared latent KV (Hkv == 1, v aliasing k), Dqk == 576,
 *                   Dv == 512, Hq % 64 == 0, sink none / null_logit;
 *          BLOCKSEL Dqk == Dv == 128, Hq / Hkv == 4, block_size == 64, and
 *                   Hkv % Hidx == 0 (the query heads of one kv head share one
 *                   index head).
 *   ATTN_SINK_KEY0_BIAS with ATTN_MASK_TOPK is rejected with ATTN_ERR_UNSUPPORTED.
 *
 * Device-data preconditions (not checked; checking would need a host sync):
 *   cu_seqlens is non-decreasing, starts at 0 and ends at T; block_sel entries
 *   are 0 or 1 (any non-zero byte counts as selected); q, k, v hold finite
 *   values.  Top-k entries outside [0, Tk) are padding, so any int32 is safe.
 *
 * Returns ATTN_OK or a negative attn_status.  T == 0 returns ATTN_OK without
 * launching.
 */
int attn_sink_fwd(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                  const int32_t* cu_seqlens, int32_t num_seqs,
                  int32_t mask_kind, const attn_mask_arg* mask,
                  const float* sinks, int32_t sink_mode, float scale,
                  const attn_tensor* out, float* lse, hipStream_t stream);

/*
 * attn_sink_check -- the host-side argument validation of attn_sink_fwd,
 * without touching the device: same arguments (no stream), same return code
 * attn_sink_fwd would give before launching.  Safe to call on a machine
 * without a GPU.
 */
int attn_sink_check(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                    const int32_t* cu_seqlens, int32_t num_seqs,
                    int32_t mask_kind, const attn_mask_arg* mask,
                    const float* sinks, int32_t sink_mode, float scale,
                    const attn_tensor* out, const float* lse);

/*
 * attn_sink_key0_correct -- the UNFUSED key-0 sink: a comparator for the
 * fused ATTN_SINK_KEY0_BIAS path, after the closed-form correction paragraph of
 * "[Bugfix][MiMo] Apply vision attention sinks in the window attention path".
 *
 * Takes out / lse of a WINDOW attention computed with ATTN_SINK_NONE (same
 * q, k, v, cu_seqlens, window and scale) and rewrites in place the rows i with
 * i - start(i) <= window, the only rows whose window holds their sequence's
 * first key k0 = k[start(i)] (v0 likewise):
 *     p0   = exp(scale * q[i, h, :] . k0[h / (Hq/Hkv), :] - lse[h, i])
 *     c    = p0 * (exp(sinks[h]) - 1)
 *     out' = (out + c * v0) / (1 + c),     lse' = lse + log1p(c)
 * -- the ATTN_SINK_KEY0_BIAS result up to rounding.  Other rows are neither
 * read nor written.
 *   q, k, v, out  as for attn_sink_fwd with ATTN_MASK_WINDOW (bf16 or f32,
 *                 T == Tk); Dqk and Dv must be whole 16-byte chunks
 *   out, lse      device; read and overwritten (affected rows only)
 *   sinks         device f32 [Hq], required; finite values
 *   num_seqs, window, scale: as for attn_sink_fwd
 * One kernel of num_seqs * (window + 1) x ceil(Hq / 4) workgroups.  Same error
 * codes as attn_sink_fwd (ATTN_ERR_UNSUPPORTED for a head dim that is not a
 * whole number of 16-byte chunks).
 */
int attn_sink_key0_correct(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                           const int32_t* cu_seqlens, int32_t num_seqs, int32_t window,
                           const float* sinks, float scale, const attn_tensor* out, float* lse,
                           hipStream_t stream);

/* Host-side validation of attn_sink_key0_correct only (no device access). */
int attn_sink_key0_correct_check(const attn_tensor* q, const attn_tensor* k, const attn_tensor* v,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t window,
                                 const float* sinks, float scale, const attn_tensor* out,
                                 const float* lse);

/* Most partial results attn_sink_merge accepts in one call. */
#define ATTN_SINK_MERGE_MAX_PARTS 8

/*
 * attn_sink_merge -- merges partial results over DISJOINT key sets of the same
 * query rows into the result over their union, then folds in a null-logit
 * sink once (the LSE-weighted merge the MiMo page's LSE paragraph relies on
 * for merge_attn_states; the DeepSeek-V4 page's Implementation paragraph for
 * folding the sink after all keys: the selected-only LSE makes this exact).
 * With P partials (out_p, lse_p), for every row i and head h:
 *     lse = log sum_p exp(lse_p),   out = sum_p exp(lse_p - lse) out_p
 *     ATTN_SINK_NULL_LOGIT: out *= 1 / (1 + exp(sinks[h] - lse)); lse unchanged
 * Partials with lse_p = -inf (empty key set) carry no weight; a row whose
 * partials are all empty gets out = 0, lse = -inf.  The partials are meant to
 * come from attn_sink_fwd calls with ATTN_SINK_NONE over a split key set
 * (e.g. column ranges of a top-k list, or of a cache split across devices).
 *   parts_out  host array of num_parts descriptors, each [T, Hq, Dv], dtype of out
 *   parts_lse  host array of num_parts device pointers, each dense f32 [Hq, T]
 *   num_parts  1 .. ATTN_SINK_MERGE_MAX_PARTS
 *   sinks      device f32 [Hq]; required for ATTN_SINK_NULL_LOGIT
 *   sink_mode  ATTN_SINK_NONE or ATTN_SINK_NULL_LOGIT (ATTN_SINK_KEY0_BIAS
 *              returns ATTN_ERR_UNSUPPORTED: that bias belongs to the part
 *              holding key 0)
 *   out        [T, Hq, Dv] bf16 or f32, Dv a whole number of 16-byte chunks;
 *   lse        device f32 [Hq, T]; both fully written, and neither may be one
 *              of the partial buffers (ATTN_ERR_RANGE) or overlap them
 * One kernel launch.  Errors as for attn_sink_fwd.
 */
int attn_sink_merge(const attn_tensor* parts_out, const float* const* parts_lse, int32_t num_parts,
                    const float* sinks, int32_t sink_mode, const attn_tensor* out, float* lse,
                    hipStream_t stream);

/* Host-side validation of attn_sink_merge only (no device access). */
int attn_sink_merge_check(const attn_tensor* parts_out, const float* const* parts_lse,
                          int32_t num_parts, const float* sinks, int32_t sink_mode,
                          const attn_tensor* out, const float* lse);

/*
 * Context-parallel reorder primitives (NeMo AutoModel "cp_sparse_attn" API
 * page: cp_load_balanced_global_slots, order_by_positions /
 * restore_by_positions, cp_document_ids).  Under causal context parallelism a
 * rank holds a non-contiguous, load-balanced part of the sequence; before a
 * block-sparse layer can attend over the global sequence, K/V gathered from
 * every rank are put into global token order, and the packed position ids
 * give the documents.  Each call is one kernel launch on `stream`; integer and
 * byte results are exact.
 *
 * attn_sink_cp_slots -- global slot index of every local slot: the sequence of
 * T = cp_size * t_local tokens is cut into 2 * cp_size chunks of t_local / 2,
 * and rank r holds chunks r and 2 * cp_size - 1 - r, in that order.
 *   rank   0 .. cp_size - 1: writes t_local slots of that rank;
 *          -1: writes cp_size * t_local slots, rank-major (the order of an
 *          all-gather of the shards)
 *   slots  device int64, that many entries
 * ATTN_ERR_RANGE if cp_size < 1, t_local is odd or negative, or rank is out
 * of range.
 */
int attn_sink_cp_slots(int32_t cp_size, int64_t t_local, int32_t rank, int64_t* slots, hipStream_t stream);
int attn_sink_cp_slots_check(int32_t cp_size, int64_t t_local, int32_t rank, const int64_t* slots);

/*
 * attn_sink_cp_permute_rows -- moves whole rows (everything past dim 0) of a
 * rank 1..4 tensor:
 *   scatter == 1: dst[index[i]] = src[i]   (order_by_positions: gathered rows,
 *                 index = their global positions -> global token order)
 *   scatter == 0: dst[i] = src[index[i]]   (restore_by_positions: global-ordered
 *                 rows -> the rows at the given positions, in that order)
 * for i < n; src (scatter) or dst (gather) has n rows.  index: device int64
 * [n].  With scatter, an index outside [0, dst rows) drops that row; with
 * gather, an index outside [0, src rows) writes a zero row.  For a permutation
 * the two are inverse to each other.  Rows must be dense; rows move in 16-,
 * 8- or 4-byte chunks, the widest dividing the row length, the row strides and
 * the base addresses (none: ATTN_ERR_UNSUPPORTED).  src and dst share dtype
 * and row shape and must not overlap (the same buffer gives ATTN_ERR_RANGE).
 * Duplicate scatter targets are a caller error (one of the rows wins).
 */
int attn_sink_cp_permute_rows(const attn_tensor* src, const int64_t* index, int64_t n, int32_t scatter,
                              const attn_tensor* dst, hipStream_t stream);
int attn_sink_cp_permute_rows_check(const attn_tensor* src, const int64_t* index, int64_t n, int32_t scatter,
                                    const attn_tensor* dst);

/*
 * attn_sink_cp_documents -- from global-ordered position ids (device int64
 * [T]) of packed documents:
 *   doc_ids     device int32 [T] or NULL: cumsum(positions == 0) - 1 (the
 *               page's cp_document_ids; -1 before the first position-0 token)
 *   cu_seqlens  device int32 [max_docs + 1] or NULL: segment boundaries for
 *               attn_sink_fwd -- 0, every later index whose position is 0,
 *               then T (token 0 always opens a segment, so with positions[0]
 *               == 0 the segments are exactly the documents)
 *   num_docs    device int32 scalar or NULL: number of segments.  If it
 *               exceeds max_docs only the first max_docs boundaries are
 *               written and T is not.
 * One workgroup scans the positions (one pass, 16384 per step).
 */
int attn_sink_cp_documents(const int64_t* positions, int64_t T, int32_t* doc_ids, int32_t* cu_seqlens,
                           int32_t max_docs, int32_t* num_docs, hipStream_t stream);
int attn_sink_cp_documents_check(const int64_t* positions, int64_t T, const int32_t* doc_ids,
                                 const int32_t* cu_seqlens, int32_t max_docs, const int32_t* num_docs);

/*
 * attn_sink_mla_decode_fp8 -- sparse-MLA decode over an fp8 latent KV cache
 * (the decode call site of "Apply DeepSeek-V4 attn_sink in the XPU sparse-MLA
 * Triton kernel"; the sink fold of its Implementation paragraph).  For every
 * query row i and head h, with K[j] = fp8(kv[j, 0, :]) * kv_scale[j] (576
 * values) and V[j] = the first 512 of them:
 *     out[i, h, :] = sum_j e^{l_j} V[j] / (sum_j e^{l_j} [+ e^{sinks[h]}])
 *     l_j = scale * q[i, h, :] . K[j]  over the valid entries of topk_idx[i, :]
 *     lse[h, i] = log sum_j e^{l_j}  (selected keys only)
 * The page names the fp8 cache but not its encoding; this entry point reads
 * it as OCP e4m3 values, 576 per row, with one fp32 scale per row.
 *   q          bf16 [T, Hq, 576], Hq a multiple of 64
 *   kv         ATTN_DTYPE_FP8_E4M3 [Tk, 1, 576]; row stride a multiple of 16 B
 *   kv_scale   device f32 [Tk]
 *   topk_idx   int32 [T, topk]; entries outside [0, Tk) are padding
 *   sink_mode  ATTN_SINK_NONE or ATTN_SINK_NULL_LOGIT (sinks: device f32 [Hq])
 *   out        bf16 [T, Hq, 512];  lse: device f32 [Hq, T]
 *   workspace  device memory of at least the size reported by
 *              attn_sink_mla_decode_fp8_workspace for (T, Hq, topk), 16-byte
 *              aligned; caller-owned scratch, overwritten by every call, so
 *              calls that share a workspace must not run concurrently
 * Few query rows leave the GPU idle, so each row's list is cut into pieces
 * computed by separate workgroups (fp32 partial results in the workspace) and
 * a second kernel merges them and folds the sink in once: two kernel launches
 * on `stream`.  Errors as for attn_sink_fwd; ATTN_ERR_RANGE for a workspace
 * that is too small.
 */
int attn_sink_mla_decode_fp8(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                             const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode, float scale,
                             const attn_tensor* out, float* lse, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream);
int attn_sink_mla_decode_fp8_check(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                                   const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode, float scale,
                                   const attn_tensor* out, const float* lse, const void* workspace,
                                   int64_t workspace_bytes);
/* Workspace bytes attn_sink_mla_decode_fp8 needs for T rows, Hq heads and
 * top-k lists of length topk (host-only; ATTN_ERR_RANGE if Hq is not a
 * positive multiple of 64). */
int attn_sink_mla_decode_fp8_workspace(int64_t T, int64_t Hq, int64_t topk, int64_t* bytes);

/*
 * attn_sink_mla_decode_fp8_noalloc -- the same decode as
 * attn_sink_mla_decode_fp8 (same arguments and results, same two kernels),
 * for callers that cannot allocate or pass device memory around: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace and allocates nothing; its fp32 partial results go
 * to a static device array of the library (ATTN_SINK_DECODE_SCRATCH_BYTES
 * per GPU, held from the library's load until the process ends).  The
 * scratch of the CURRENT device is used: call it with the device current
 * that `stream` belongs to.  Every call on one GPU shares that array, so
 * calls that overlap on one GPU (other streams, other host threads) race;
 * serialise them.  A call whose partials need more than the limit (see
 * attn_sink_mla_decode_fp8_workspace for the size) returns ATTN_ERR_RANGE
 * before touching the device; otherwise errors as for attn_sink_mla_decode_fp8.
 */
#define ATTN_SINK_DECODE_SCRATCH_BYTES ((int64_t)96 << 20)
int attn_sink_mla_decode_fp8_noalloc(const attn_tensor* q, const attn_tensor* kv, const float* kv_scale,
                                     const attn_tensor* topk_idx, const float* sinks, int32_t sink_mode, float scale,
                                     const attn_tensor* out, float* lse, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_sink_strerror(int status);

/* ATTN_SINK_ABI_VERSION of the built library. */
int attn_sink_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H */
