/*
 * hysparse.h - C ABI of the HySparse hybrid-block attention library for one
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages: the HySparse abstract; the intelliparadigm HySparse
 * article sections 2.1, 2.2 and 3.1; the Baidu article "Sparse Evolution of
 * Hybrid Attention Architectures", section "Fine-Grained Sparse Attention:
 * Indexer + Top-K"):
 *
 *   full layer    O[b,i,h]   = sum_j softmax_j(tau * q.k_j, j <= pos(i)) v_j
 *                 S[b,g,n,j] = sum over heads h of KV group g and queries i of
 *                              score block n of P[b,h,i,j]   (importance score)
 *   top-K         idx[b,g,n] = the K largest S[b,g,n,j] over j <= last(n)
 *   sparse layer  out = sigmoid(w_h) * o_global + (1 - sigmoid(w_h)) * o_local
 *                 o_global: softmax attention over {j in idx[b,g,n] : j <= pos(i)}
 *                 o_local:  softmax attention over the W keys [pos(i)-W+1, pos(i)]
 *                 both on the full layer's K and V (the cache is shared, read only)
 *
 * Conventions shared by every entry point
 *   - pos(i) = kv_len - q_len + i; tau = 1/sqrt(head_dim) unless desc.scale > 0;
 *     query head h uses KV head h / (n_q_heads / n_kv_heads).
 *   - Score blocks: n = i / score_block, NB = ceil(q_len / score_block),
 *     last(n) = pos(min((n+1)*score_block, q_len) - 1).  score_block is 1 or 64.
 *   - Top-K order: the float32 bit pattern u is mapped to a key that is
 *     u ^ 0xFFFFFFFF for negative values and u ^ 0x80000000 otherwise; larger
 *     key first, lower index first among equal keys.  Index rows are sorted
 *     ascending and padded with -1 when fewer than K candidates exist.
 *   - Memory: every pointer argument except host arrays explicitly marked
 *     "host" is device memory owned by the caller.  The library allocates
 *     nothing and keeps no state between calls; all scratch comes from the
 *     caller's workspace, sized by hysparse_workspace_bytes /
 *     hysparse_topk_workspace_bytes.  A workspace must not be shared by calls
 *     that may run concurrently.
 *   - Layout: q, k, v are strided by desc (elements; the head_dim axis is
 *     contiguous).  Outputs are dense: out [B, Tq, Hq, D] in desc.dtype,
 *     lse [B, Hq, Tq] float32 (natural log), scores [B, Hkv, NB, Tkv] float32,
 *     idx [B, Hkv, NB, K] int32.  Base pointers must be 16-byte aligned and
 *     the batch/token/head strides multiples of 16 bytes.
 *   - Errors: every argument is checked on the host before anything is
 *     enqueued; on error nothing is launched and a status != 0 is returned
 *     (hysparse_last_error() gives the detail).  After launching, a HIP launch
 *     error maps to HYS_ERR_HIP.  Device-side faults surface at the caller's
 *     next synchronisation.  Nothing throws across this interface.
 *   - Asynchrony: all work is enqueued on `stream` (0 = the null stream); the
 *     call returns without waiting.
 *   - Supported shapes: head_dim 64 or 128; n_q_heads % n_kv_heads == 0 with
 *     1 <= n_q_heads / n_kv_heads <= 16; 1 <= q_len <= kv_len; dtype bf16 or
 *     float32.  NaN or Inf in q, k or v is outside the contract.
 */
#ifndef HYSPARSE_H
#define HYSPARSE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hys_status;

enum {
  HYS_OK = 0,
  HYS_ERR_NULL_PTR = 1,     /* a required pointer is NULL                     */
  HYS_ERR_BAD_SHAPE = 2,    /* inconsistent or out-of-range sizes             */
  HYS_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head_dim, dtype ...) */
  HYS_ERR_ALIGN = 4,        /* a pointer or stride is not 16-byte aligned     */
  HYS_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required     */
  HYS_ERR_HIP = 6           /* the HIP runtime reported an error              */
};

typedef enum { HYS_F32 = 0, HYS_BF16 = 1 } hys_dtype;

/* Attention problem shared by the entry points.  Strides are in elements for
 * the (batch, token, head) axes of q ([B, Tq, Hq, D]) and of k and v
 * ([B, Tkv, Hkv, D]; k and v share strides). */
typedef struct {
  int32_t batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim;
  int32_t dtype;          /* hys_dtype of q, k, v and of the attention outputs */
  float scale;            /* softmax scale; <= 0 selects 1/sqrt(head_dim)      */
  int64_t q_stride[3];
  int64_t kv_stride[3];
} hys_attn_desc;

/* Operation ids for hysparse_workspace_bytes. */
enum { HYS_OP_FULL = 0, HYS_OP_TOPK = 1, HYS_OP_SPARSE = 2, HYS_OP_HYBRID = 3 };

/*
 * Full-attention layer with importance-score emission (HySparse abstract: the
 * full layer is the oracle that selects tokens; intelliparadigm article 3.1:
 * its importance scores are reused by the following sparse layers).
 *
 *   q, k, v      inputs laid out by desc.
 *   score_block  1 (one score row per query) or 64 (one per 64-query block).
 *   out          [B, Tq, Hq, D] desc.dtype, written.
 *   lse          [B, Hq, Tq] float32 log-sum-exp of the scaled logits, or NULL.
 *   scores       [B, Hkv, NB, Tkv] float32, written in full (0 past last(n)).
 *                Formed from fp32 logits of the stored inputs.  With
 *                q_len 1 each head's probability passes between two kernels
 *                as an fp32 value (fp32 inputs) or an fp32 value rounded to
 *                16 significant bits (bf16 inputs), a relative error of at
 *                most 2^-16 per term.
 *   ws/ws_bytes  workspace of at least hysparse_workspace_bytes(HYS_OP_FULL, ...).
 */
hys_status hysparse_full_attn_scores(const hys_attn_desc* desc, const void* q, const void* k,
                                     const void* v, int32_t score_block, void* out, float* lse,
                                     float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Top-K select over score rows (Baidu article, "Fine-Grained Sparse Attention:
 * Indexer + Top-K": keep the K best positions per query; intelliparadigm
 * article 2.2: TopK indices of the preceding full layer).
 *
 *   scores       float32 rows; row r starts at scores + r * row_stride.
 *   n_rows       number of rows (>= 0); row_len = columns per row (>= 1).
 *   row_stride   elements between rows, >= row_len, multiple of 4.
 *   valid_len    int32 [n_rows] candidates per row (clamped to [0, row_len]),
 *                or NULL for row_len everywhere.
 *   k            K >= 1.
 *   idx          int32 [n_rows, k], written: ascending indices, -1 padded.
 *   ws/ws_bytes  at least hysparse_topk_workspace_bytes(n_rows, row_len, k)
 *                bytes.  That size is 0 (ws may be NULL) unless there are
 *                fewer than 256 rows longer than 12288 keys: such rows are
 *                filtered in parts by several workgroups each, whose
 *                candidates go to the workspace, a slot of min(part length,
 *                12288) keys and indices per part (16 rows of 131072 keys:
 *                32 parts of 4096, about 17 MB).  A NULL or smaller ws then returns
 *                HYS_ERR_WORKSPACE.
 * Results are bit-exact functions of the input bits (no atomics-order effects).
 */
hys_status hysparse_topk(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride,
                         const int32_t* valid_len, int32_t k, int32_t* idx, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/*
 * Sparse layer (intelliparadigm article 2.2: global branch on the shared KV at
 * the TopK indices, 128-token sliding-window branch, sigmoid-gated sum;
 * Baidu article pseudocode: gather k_cache[idx], v_cache[idx], then softmax
 * attention).  k and v are the full layer's cache and are only read.
 *
 *   q            this layer's queries, laid out by desc.
 *   idx          int32 [B, Hkv, NB, k_top]; entries < 0 are skipped, entries
 *                > pos(i) are masked per query, duplicates are not allowed.
 *   window       W >= 1 keys ending at each query's own position.
 *   gate_logits  float32 [Hq] (device); +-inf give gate 1 / 0 exactly.
 *   out          [B, Tq, Hq, D] desc.dtype, written.
 */
hys_status hysparse_sparse_attn(const hys_attn_desc* desc, const void* q, const void* k,
                                const void* v, const int32_t* idx, int32_t k_top,
                                int32_t score_block, int32_t window, const float* gate_logits,
                                void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Sparse layer with one gate logit per token and head (the input-dependent
 * reading of the learnable sigmoid gate of intelliparadigm article 2.2,
 * g = sigmoid(x . w_h) with the projection x . w_h computed by the caller).
 * The logit of (batch b, query i, query head h) is
 *   gate_logits[b * gate_stride_b + i * gate_stride_t + h];
 * strides (Tq * Hq, Hq) read a contiguous [B, Tq, Hq] float32 tensor, strides
 * (0, 0) one logit per head (exactly hysparse_sparse_attn).  Everything else
 * as hysparse_sparse_attn.  Errors: negative strides -> HYS_ERR_BAD_SHAPE.
 */
hys_status hysparse_sparse_attn_token_gate(const hys_attn_desc* desc, const void* q, const void* k,
                                           const void* v, const int32_t* idx, int32_t k_top,
                                           int32_t score_block, int32_t window, const float* gate_logits,
                                           int64_t gate_stride_b, int64_t gate_stride_t, void* out, void* ws,
                                           size_t ws_bytes, hipStream_t stream);

/*
 * Keys and values of a sparse layer's own window branch (the reading in which
 * each sparse layer maintains its own 128-token window, intelliparadigm
 * article 2.2), in desc.dtype with head_dim contiguous.  Position p of batch b
 * and KV head h is row (ring > 0 ? p % ring : p) of the buffer:
 *   k, v     16-byte aligned, caller-owned, read.
 *   stride   element strides of the (batch, row, head) axes, multiples of 16 bytes.
 *   ring     > 0: a ring of `ring` rows holding the most recent positions
 *            (decode: ring >= window; prefill: ring >= window + q_len - 1 so
 *            that every position a call reads has its own row); 0: rows are
 *            positions (the buffer spans at least kv_len rows).
 * The caller keeps the buffer current (hysparse_append_kv writes a row).
 */
typedef struct {
  const void* k;
  const void* v;
  int64_t stride[3];
  int32_t ring;
} hys_window_kv;

/*
 * The general sparse layer: gate logits as in hysparse_sparse_attn_token_gate
 * (strides 0, 0: one logit per head) and, when own_window is not NULL, the
 * window branch over the layer's own window keys/values instead of the shared
 * cache (the global branch always reads the shared cache at the indices).
 * Everything else as hysparse_sparse_attn.  Errors: negative gate strides, a
 * ring shorter than the positions one call reads -> HYS_ERR_BAD_SHAPE;
 * misaligned window buffers or strides -> HYS_ERR_ALIGN.
 */
hys_status hysparse_sparse_attn_ex(const hys_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const int32_t* idx, int32_t k_top, int32_t score_block, int32_t window,
                                   const float* gate_logits, int64_t gate_stride_b, int64_t gate_stride_t,
                                   const hys_window_kv* own_window, void* out, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * hysparse_sparse_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, outputs and errors as
 * hysparse_sparse_attn, minus ws/ws_bytes: the split partial states of the
 * one-query-row path (score_block 1 or q_len 1) go to a fixed scratch array
 * inside the library, hysparse_noalloc_scratch_bytes() bytes (16 MiB) per
 * GPU, held from the first call on that GPU until the process ends.  The
 * scratch used is that of the device current at the call, so `stream` must
 * belong to the current device.  Calls needing more scratch than that (what
 * hysparse_workspace_bytes(HYS_OP_SPARSE, ...) returns) fail with
 * HYS_ERR_WORKSPACE before anything is launched.  The call allocates nothing.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, or graphs replayed concurrently) race and must
 * not be issued; calls ordered on one stream are safe.  Nothing in the
 * scratch needs to start at zero (each call writes every partial it reads).
 */
hys_status hysparse_sparse_attn_noalloc(const hys_attn_desc* desc, const void* q, const void* k,
                                        const void* v, const int32_t* idx, int32_t k_top,
                                        int32_t score_block, int32_t window, const float* gate_logits,
                                        void* out, hipStream_t stream);

/* Bytes of the fixed scratch behind hysparse_sparse_attn_noalloc. */
size_t hysparse_noalloc_scratch_bytes(void);

/*
 * One hybrid block (intelliparadigm article 2.1 and 3.1): the full layer on
 * q_full, top-K over its scores, then n_sparse sparse layers that reuse its
 * k, v and indices, each with its own queries and gate logits.
 *
 *   q_sparse     host array of n_sparse device pointers, each laid out by desc.
 *   gate_logits  float32 [n_sparse, Hq] (device).
 *   out_full     [B, Tq, Hq, D]; out_sparse: host array of n_sparse device
 *                pointers to [B, Tq, Hq, D] outputs.
 *   lse, scores, idx  optional outputs (NULL: kept in the workspace only).
 */
hys_status hysparse_hybrid_block(const hys_attn_desc* desc, const void* q_full, const void* k,
                                 const void* v, int32_t n_sparse, const void* const* q_sparse,
                                 const float* gate_logits, int32_t k_top, int32_t score_block,
                                 int32_t window, void* out_full, void* const* out_sparse,
                                 float* lse, float* scores, int32_t* idx, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * Hierarchical selection for decode (q_len 1), a variant of the top-K step
 * (HISA abstract: a block-level coarse filter over pooled block
 * representatives, then token-level selection inside the surviving blocks;
 * Baidu article, "Configuration Considerations": pooled representations for
 * scoring).
 *
 *   1. pooled keys: the mean of each run of `block` consecutive keys of a KV
 *      group (the last run may be shorter);
 *   2. block score: softmax over the pooled keys of each query head of the
 *      group (scale as desc), summed over the group's heads;
 *   3. the n_keep best blocks by the top-K order rule;
 *   4. the k_top best tokens of those blocks by the full layer's scores.
 *
 *   q, k          as for hysparse_full_attn_scores (q_len must be 1).
 *   scores        float32 [B, Hkv, 1, Tkv]: the full layer's scores.
 *   block_scores  float32 [B, Hkv, ceil(Tkv/block)] or NULL (workspace only).
 *   blocks        int32 [B, Hkv, n_keep] kept block ids, ascending, -1
 *                 padded; or NULL.
 *   idx           int32 [B, Hkv, 1, k_top] token indices, ascending, -1 padded.
 *   ws/ws_bytes   at least hysparse_hier_workspace_bytes(desc, block, n_keep, k_top).
 */
hys_status hysparse_hier_select(const hys_attn_desc* desc, const void* q, const void* k,
                                const float* scores, int32_t block, int32_t n_keep, int32_t k_top,
                                float* block_scores, int32_t* blocks, int32_t* idx, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * Pooled keys kept beside the cache, for hierarchical selection in a decode
 * loop.  The pooled key of a complete block does not change as the cache
 * grows (intelliparadigm article section 3.1: only the full layers update the
 * cache), so a caller pools every block once and, after each
 * hysparse_append_kv, refreshes only the blocks the new tokens touch.
 *
 * hysparse_hier_pool writes, for blocks m in [m_begin, m_end),
 *   kbar[b, m, g, :] = mean of keys [m * block, min((m + 1) * block, kv_len))
 * of KV group g, in fp32.  desc's kv fields describe the cache as for
 * hysparse_append_kv (kv_len: the tokens it holds now); its query fields are
 * not read.
 *
 *   k             the cache's keys, 16-byte aligned, read.
 *   kbar          float32 [B, kbar_blocks, Hkv, D] (batch stride kbar_blocks
 *                 * Hkv * D floats), 16-byte aligned, caller-owned, written
 *                 for the given blocks only.
 *   kbar_blocks   blocks held per batch entry: >= ceil(kv_len / block) (the
 *                 cache capacity in blocks, so the array outlives growth).
 *   Errors: block < 1, m_begin < 0, m_end < m_begin, m_end > ceil(kv_len /
 *   block) or kbar_blocks too small -> HYS_ERR_BAD_SHAPE; no workspace.
 *
 * hysparse_hier_select_pooled is hysparse_hier_select with step 1 replaced by
 * the given pooled keys (all ceil(kv_len / block) blocks valid); its other
 * arguments, outputs and workspace are those of hysparse_hier_select, and
 * with kbar from hysparse_hier_pool over every block its outputs equal
 * hysparse_hier_select's bit for bit.
 */
hys_status hysparse_hier_pool(const hys_attn_desc* desc, const void* k, int32_t block, int32_t m_begin, int32_t m_end,
                              float* kbar, int32_t kbar_blocks, hipStream_t stream);
hys_status hysparse_hier_select_pooled(const hys_attn_desc* desc, const void* q, const float* kbar,
                                       int32_t kbar_blocks, const float* scores, int32_t block, int32_t n_keep,
                                       int32_t k_top, float* block_scores, int32_t* blocks, int32_t* idx, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/*
 * KV-cache append (intelliparadigm article section 3.1: only the full layers
 * update the cache; the sparse layers read it).  Copies n_new new rows of keys
 * and values, each [B, n_new, Hkv, D] contiguous in desc.dtype, into the cache
 * at token positions [pos, pos + n_new) of every batch entry and KV head.  The
 * cache is described by desc's kv fields: kv_len is its capacity in tokens,
 * kv_stride its (batch, token, head) strides; batch, n_kv_heads, head_dim and
 * dtype as for the other calls.  desc's query fields are not read.  The full
 * layer then runs on the cache with kv_len = pos + n_new (a decode step:
 * n_new = 1; chunked prefill: n_new = the chunk length).
 *
 *   k_new, v_new      new rows, 16-byte aligned, caller-owned, read.
 *   k_cache, v_cache  cache, 16-byte aligned, caller-owned, written.
 *   Errors: NULL pointers -> HYS_ERR_NULL_PTR; n_new < 1, pos < 0 or
 *   pos + n_new > kv_len -> HYS_ERR_BAD_SHAPE; no workspace is needed.
 */
hys_status hysparse_append_kv(const hys_attn_desc* desc, const void* k_new, const void* v_new, int32_t n_new,
                              int32_t pos, void* k_cache, void* v_cache, hipStream_t stream);

/* Workspace bytes for hysparse_hier_select (0 for invalid arguments). */
size_t hysparse_hier_workspace_bytes(const hys_attn_desc* desc, int32_t block, int32_t n_keep,
                                     int32_t k_top);

/* Workspace bytes for op (HYS_OP_*) on desc; k_top and window are ignored
 * where they do not apply.  For HYS_OP_HYBRID the figure covers scores and
 * idx kept in the workspace (the NULL-output case) and any n_sparse.
 * Returns 0 for invalid arguments. */
size_t hysparse_workspace_bytes(int32_t op, const hys_attn_desc* desc, int32_t score_block,
                                int32_t k_top, int32_t window);

/* Workspace bytes for hysparse_topk. */
size_t hysparse_topk_workspace_bytes(int64_t n_rows, int32_t row_len, int32_t k);

/* Static description of a status code. */
const char* hysparse_status_string(hys_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* hysparse_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t hysparse_version(void);

/*
 * Index-set check, a debugging aid for callers that build index rows for the
 * sparse layer themselves (the sparse layer requires distinct entries: a key
 * listed twice would enter the global branch's softmax twice; see
 * hysparse_sparse_attn).  Nothing traps; for each row r of idx (int32
 * [n_rows, k], rows k apart) status[r] (int32, device) gets the OR of:
 *   HYS_IDX_DUPLICATE     a non-negative entry below row_len appears twice;
 *   HYS_IDX_OUT_OF_RANGE  an entry is below -1, or not below the row's
 *                         candidate count (valid_len[r] clamped to
 *                         [0, row_len], or row_len when valid_len is NULL);
 *                         the sparse layer skips or masks such entries;
 *   HYS_IDX_ORDER         the row is not in the form hysparse_topk writes
 *                         (non-negative entries strictly ascending, -1
 *                         padding only after them); the sparse layer accepts
 *                         any order.
 * A row written by hysparse_topk has status 0.  Requires 1 <= row_len <=
 * 524288 (HYS_ERR_UNSUPPORTED otherwise), k >= 1, 0 <= n_rows < 2^31.
 */
enum { HYS_IDX_DUPLICATE = 1, HYS_IDX_OUT_OF_RANGE = 2, HYS_IDX_ORDER = 4 };
hys_status hysparse_check_indices(const int32_t* idx, int64_t n_rows, int32_t k, int32_t row_len,
                                  const int32_t* valid_len, int32_t* status, hipStream_t stream);

/*
 * Measurement helpers (not part of the computation): size-matched bandwidth
 * ceilings.  A decode-time sparse layer moves a few tens of MB per launch,
 * too little for one launch to reach the HBM peak; these kernels give what a
 * launch of the same size reaches with nothing else to do (Baidu article,
 * "Key Engineering Considerations": decoding is bound by memory bandwidth).
 * Both only read their inputs and write one word per workgroup into ws.
 *
 * hysparse_ceiling_stream_read  reads n_bytes (a multiple of 16) from the
 *                               16-byte aligned device buffer p.
 * hysparse_ceiling_gather       reads row_bytes (a multiple of 16, <= 256)
 *                               at k + rows[r] * row_stride_bytes and at
 *                               v + rows[r] * row_stride_bytes for every
 *                               r < n_rows whose rows[r] lies in
 *                               [0, n_buffer_rows) (others are skipped),
 *                               the row indices loaded first.
 * ws/ws_bytes: at least hysparse_ceiling_workspace_bytes(n_bytes, n_rows).
 */
size_t hysparse_ceiling_workspace_bytes(int64_t n_bytes, int64_t n_rows);
hys_status hysparse_ceiling_stream_read(const void* p, int64_t n_bytes, void* ws, size_t ws_bytes,
                                        hipStream_t stream);
hys_status hysparse_ceiling_gather(const void* k, const void* v, int64_t row_stride_bytes, int64_t n_buffer_rows,
                                   const int32_t* rows, int64_t n_rows, int32_t row_bytes, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * Kernel-level timing hook for profilers (not part of the computation).
 * While a trace is active on the calling thread, the library records, on the
 * launch stream, events[2i] just before and events[2i+1] just after the i-th
 * kernel it launches, for as long as 2i+1 < capacity.  `events` is a host
 * array of events the caller created (hipEventCreate) and keeps alive until
 * the recorded work has completed.  This is the library's only per-thread
 * state besides the last-error text.
 *   hysparse_trace_begin  starts (or restarts) the trace; events NULL stops it.
 *   hysparse_trace_end    stops it and returns the number of kernels traced.
 *   hysparse_trace_name   static name of the i-th traced kernel ("" if none);
 *                         valid until the next hysparse_trace_begin.
 */
void hysparse_trace_begin(hipEvent_t* events, int32_t capacity);
int32_t hysparse_trace_end(void);
const char* hysparse_trace_name(int32_t i);

#ifdef __cplusplus
}
#endif

#endif /* HYSPARSE_H */
