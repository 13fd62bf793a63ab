/*
 * msgl.h — C ABI of the paged-KV attention library (gfx950 / MI355X).
 *
 * Operations (all from the mini-sglang pages):
 *   msgl_store_kv      scatter new K/V rows into the pool at out_loc
 *                      ["Mini-SGLang complete analysis", §4.4.3 (pool tensor,
 *                      flattened per layer to (slots, kv heads, head_dim)),
 *                      §4.6.7 (the attention layer stores first), §4.9.4 (the
 *                      store kernel's shape contract), §4.9.5 (vector copies)]
 *   msgl_paged_decode  one query token per request, GQA, keys gathered through
 *                      a token-granular page-table row
 *                      [same page, §1.2 (decode is memory-bound), §1.4 (paged
 *                      pool + per-request page table), §4.5.3 (GQA ratio),
 *                      §4.6.4 (table kept at page_size 1)]
 *   msgl_store_kv_paged_decode  the two above in one launch, as the
 *                      attention layer's forward runs them back to back
 *                      ["Mini-SGLang complete analysis" §4.6.7]
 *   msgl_paged_extend  causal chunked-prefill attention over a cached prefix
 *                      plus the chunk itself
 *                      ["Deep dive into mini-sglang: chunked prefill and
 *                      overlap scheduling", chunked-prefill section;
 *                      "Mini-SGLang complete analysis" §4.2.3 (cached_len /
 *                      extend_len), §4.6.5 (cu_seqlens_q)]
 *   msgl_merge_states  log-sum-exp merge of partial attention results (the
 *                      pages do not describe split-KV; the merge is the exact
 *                      identity that recombines a softmax split over disjoint
 *                      key sets)
 *   msgl_rope_cos_sin_cache, msgl_qk_norm_rope_store   the attention layer's
 *                      prologue: q/k RMSNorm, RoPE, store of K/V, fused
 *                      ["Mini-SGLang complete analysis" §4.6.7, §4.5.6]
 *   msgl_embedding_gather  token-id -> embedding-row gather with the
 *                      vocabulary-shard mask ["Mini-SGLang complete analysis",
 *                      §4.9.3 (indexing), §4.7.8 (embed_tokens sharded along
 *                      the vocabulary, masked indexing + all-reduce)]
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller.  The library
 *   never allocates, frees or synchronises; every call only enqueues work on
 *   `stream` and returns.  Buffers must stay alive and unmodified until that
 *   work has completed (the pages' rule against freeing a batch's inputs while
 *   the GPU may still read them, §4.2.5).
 * - bf16 is the only element type of K, V, q and outputs (dtype code
 *   MSGL_DTYPE_BF16); head_dim must be 128; q heads per kv head ("ratio")
 *   must be 1, 2, 4, 8 or 16.
 * - Pool layout: one layer's K (and separately V) is `[num_slots, num_kv_heads,
 *   head_dim]`, head_dim contiguous, kv heads contiguous, consecutive slots
 *   `cache_row_stride` elements apart.  Pass the layer's K and V base pointers
 *   (the pages' 6-D pool is [2][layers][pages][page_size][kv_heads][dim]).
 * - page_table: int32 `[rows, page_table_stride]`; entry (row, j) is the slot
 *   of token j of the request that owns the row.  With page_size P > 1 the
 *   caller guarantees that entries inside a page are consecutive slots; results
 *   are bit-identical to passing P = 1 for the same table.
 * - Lengths and indices that live in device memory (seq_lens, prefix_lens,
 *   extend_lens, q_offsets, req_rows, page_table entries, out_loc) are NOT
 *   range-checked in the release library: out-of-range values are undefined
 *   behaviour, as in the pages' kernels.  Host-side scalars and pointers ARE
 *   validated before any HIP call; a rejected call enqueues nothing.
 * - The debug-check library (libmsgl_debug.so, the same sources built with
 *   MSGL_DEBUG_CHECKS; msgl_debug_checks() returns 1 there) also checks them
 *   on the device before each store, decode, extend and prologue call: out_loc
 *   entries in [0, num_slots); lengths non-negative, within their declared
 *   maxima (max_seq_len, max_extend_len, max_kv_len) and the page-table width;
 *   q_offsets steps equal to extend_len; req_rows entries non-negative; every
 *   page-table entry the call would read inside the pool; for the fused store
 *   + decode, out_loc[r] equal to the slot of request r's newest key.  The
 *   check runs on the call's stream and the call WAITS for it (a debug
 *   build); on failure the call launches nothing else and returns
 *   MSGL_ERR_INDEX with the first offending request, key and value in
 *   msgl_last_error().  Not checked: that out_loc entries are distinct, and a
 *   req_rows entry past the last table row (no row count crosses the ABI).
 *   Under stream capture the checks are skipped (nothing may wait there).
 * - Return value: MSGL_OK (0) or a negative msgl_status.  No exception crosses
 *   the ABI.  msgl_last_error() returns a thread-local message for the last
 *   failure on the calling thread (including the source location).
 */
#ifndef MSGL_H
#define MSGL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msgl_status {
  MSGL_OK = 0,
  MSGL_ERR_NULL = -1,         /* a required pointer is NULL                     */
  MSGL_ERR_SHAPE = -2,        /* sizes/strides inconsistent or negative         */
  MSGL_ERR_UNSUPPORTED = -3,  /* dtype, head_dim, ratio or page_size not served */
  MSGL_ERR_ALIGN = -4,        /* pointer or stride breaks required alignment    */
  MSGL_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required     */
  MSGL_ERR_LAUNCH = -6,       /* the HIP runtime rejected a kernel launch       */
  MSGL_ERR_INDEX = -7         /* debug-check build: device index out of range   */
} msgl_status;

enum { MSGL_DTYPE_BF16 = 0, MSGL_DTYPE_F32 = 1 };
enum { MSGL_INDEX_I32 = 0, MSGL_INDEX_I64 = 1 };

/* Library version as major*10000 + minor*100 + patch. */
int msgl_version(void);

/* 1 in the debug-check library (device indices checked before each call,
 * see above), 0 in the release library. */
int msgl_debug_checks(void);

/* Static text for a status code. */
const char* msgl_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* msgl_last_error(void);

/*
 * msgl_store_kv — k_cache[out_loc[i]] = k_new[i]; v_cache[out_loc[i]] = v_new[i]
 * for i in [0, n).  A pure byte copy of one row (num_kv_heads * head_dim
 * elements) per index; every other slot is left untouched.
 *
 *   k_cache, v_cache   pool planes of one layer, [num_slots, row] elements,
 *                      slot s at offset s * cache_row_stride
 *   k_new, v_new       [n, row] elements, row i at i * new_row_stride
 *   out_loc            n indices, int32 (index_dtype = MSGL_INDEX_I32) or
 *                      int64 (MSGL_INDEX_I64); must be distinct and in
 *                      [0, num_slots)
 *   row = num_kv_heads * head_dim elements of `dtype` (bf16 or f32).
 * Vector width follows alignment: 16-byte copies when pointers, strides and
 * the row size allow, else 8, 4 or 2 bytes (never an error for alignment).
 * n == 0 enqueues nothing and returns MSGL_OK.
 */
int msgl_store_kv(void* k_cache, void* v_cache, int64_t num_slots,
                  int64_t cache_row_stride, const void* k_new, const void* v_new,
                  int64_t new_row_stride, const void* out_loc, int32_t index_dtype,
                  int64_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                  hipStream_t stream);

/*
 * msgl_paged_decode — for each request r in [0, batch) and q head h:
 *   L = seq_lens[r] (keys, INCLUDING the token just stored), row = req_rows[r]
 *   (or r when req_rows is NULL), g = h / (num_q_heads / num_kv_heads),
 *   s_j = sm_scale * dot(q[r, h], K[page_table[row, j], g]),  j in [0, L)
 *   out[r, h]  = sum_j softmax(s)_j * V[page_table[row, j], g]   (bf16)
 *   lse_out[r, h] = ln sum_j exp(s_j)                           (fp32, optional)
 * L == 0 gives out = 0 and lse = -inf.
 *
 *   out        bf16 [batch, num_q_heads, 128], contiguous
 *   lse_out    fp32 [batch, num_q_heads] or NULL
 *   q          bf16 [batch, num_q_heads, 128]; request r at r * q_row_stride
 *              elements (>= num_q_heads * 128), heads contiguous
 *   max_seq_len  host upper bound on every seq_lens[r] (sizes grid/workspace)
 *   split_tokens keys per split-KV chunk (multiple of 32), or 0 for automatic.
 *              Chunk c of request r covers keys [c*S, min((c+1)*S, L)); requests
 *              with more than one chunk are recombined with the LSE merge.
 *   workspace  device scratch of at least msgl_paged_decode_workspace_size(...)
 *              bytes (may be NULL when that size is 0); contents on entry are
 *              ignored, 256-byte alignment required.
 * Deterministic: for fixed inputs and split size the result bits do not depend
 * on scheduling, on which slots hold the keys, or on page_size.
 */
int msgl_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                      const void* k_cache, const void* v_cache, int64_t num_slots,
                      int64_t cache_row_stride, const int32_t* page_table,
                      int64_t page_table_stride, const int32_t* req_rows,
                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_seq_len, float sm_scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msgl_store_kv_paged_decode — msgl_store_kv of one new row per request
 * followed by msgl_paged_decode, in one launch ("Mini-SGLang complete
 * analysis" §4.6.7: the attention layer's forward stores the step's K/V and
 * then attends over the pool, so the newest key of every request is the row
 * just stored).  Row r of k_new / v_new ([batch, row] elements, row r at
 * r * new_row_stride, 16-byte aligned rows) is request r's new token: it is
 * written to slot out_loc[r] (int32 or int64 per index_dtype), and the
 * attention takes key seq_lens[r] - 1 of request r from that row directly,
 * so no part of the launch reads a slot another part is writing.
 * The caller guarantees, for every request r with seq_lens[r] > 0, that
 * out_loc[r] == page_table[row, seq_lens[r] - 1] and that no other request
 * of the batch has out_loc[r] among its keys (the slot was just allocated
 * for r's new token, as the pages' allocator does; shared prefix pages hold
 * cached keys only).  Then the pool and the outputs are bit-identical to
 * msgl_store_kv(n = batch) followed by msgl_paged_decode with the same
 * arguments; otherwise another request may see the slot before or after
 * the store.  Every other
 * argument, the workspace and the errors are those of the two calls
 * (k_new / v_new rows must also be 16-byte aligned: MSGL_ERR_ALIGN).
 */
int msgl_store_kv_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               void* k_cache, void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const void* k_new, const void* v_new,
                               int64_t new_row_stride, const void* out_loc, int32_t index_dtype,
                               const int32_t* page_table, int64_t page_table_stride,
                               const int32_t* req_rows, const int32_t* seq_lens, int32_t batch,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t page_size, int32_t max_seq_len, float sm_scale,
                               int32_t split_tokens, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of device memory that msgl_store_kv_paged_decode_noalloc may use for
 * its partial results (32 MiB). */
#define MSGL_DECODE_SCRATCH_BYTES (32u << 20)

/*
 * msgl_store_kv_paged_decode_noalloc — msgl_store_kv_paged_decode for
 * callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The arguments, results and errors are those of
 * msgl_store_kv_paged_decode without `workspace` / `workspace_bytes`; the
 * outputs are bit-identical to it.  The partial outputs, partial lse and
 * per-request workgroup ranges live in one static device array of
 * MSGL_DECODE_SCRATCH_BYTES inside the library (one copy per GPU, held
 * until the process ends, its address looked up once per device on the
 * first call there).  The call allocates and frees nothing and makes no
 * allocating library call.
 * Limit: a batch whose partial results need more than
 * MSGL_DECODE_SCRATCH_BYTES is rejected with MSGL_ERR_WORKSPACE before any
 * launch (in balanced mode the need is 4 * num_q_heads * (head_dim + 1) *
 * (resident workgroups + batch) bytes plus 8 per request, about 16.8 MB at
 * 64 q heads and batch 256 on a 256-CU device).
 * Every call on one GPU shares that GPU's array and nothing in it needs to
 * start at any value (each call writes every entry it later reads), but
 * calls whose work overlaps on one GPU (different streams, or host threads
 * without ordering) race on it and give undefined results.
 */
int msgl_store_kv_paged_decode_noalloc(void* out, float* lse_out, const void* q,
                                       int64_t q_row_stride, void* k_cache, void* v_cache,
                                       int64_t num_slots, int64_t cache_row_stride,
                                       const void* k_new, const void* v_new,
                                       int64_t new_row_stride, const void* out_loc,
                                       int32_t index_dtype, const int32_t* page_table,
                                       int64_t page_table_stride, const int32_t* req_rows,
                                       const int32_t* seq_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t page_size, int32_t max_seq_len,
                                       float sm_scale, int32_t split_tokens, hipStream_t stream);

/* Bytes of workspace msgl_paged_decode needs for these host-side sizes
 * (0 if no request can need more than one chunk).  The split size actually
 * used is written to *split_tokens_out when it is not NULL. */
size_t msgl_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_seq_len, int32_t split_tokens,
                                        int32_t* split_tokens_out);

/*
 * msgl_paged_extend — causal extend.  Request r has P = prefix_lens[r] cached
 * keys and E = extend_lens[r] new tokens, whose K/V were already stored into
 * the pool at page_table[row, P .. P+E-1].  Its queries are rows
 * q_offsets[r] .. q_offsets[r]+E-1 of q (q_offsets[r+1] - q_offsets[r] == E).
 * Query i (absolute position P+i) attends keys j in [0, P+i] (bottom-right
 * aligned causal mask); with P == 0 this is ordinary causal prefill.
 *
 *   out        bf16 [T, num_q_heads, 128] contiguous, T = q_offsets[batch]
 *   lse_out    fp32 [T, num_q_heads] or NULL
 *   q          bf16 [T, num_q_heads, 128], row t at t * q_row_stride elements
 *   max_extend_len, max_kv_len   host upper bounds on E and P + E
 *   causal     must be 1 (the only mode the method uses)
 *   workspace  optional, device memory of at least
 *              msgl_paged_extend_workspace_size(...) bytes, 16-byte aligned,
 *              owned by the caller and overwritten by the call.  With it and
 *              batch > 1, a planning pass orders the (request, query tile)
 *              work items longest first before the attention pass; with
 *              NULL (or one request, whose tiles are already in that order)
 *              the items run last query tile first.  The results are
 *              bit-identical either way; only the load balance differs.  A
 *              non-NULL workspace smaller than required is
 *              MSGL_ERR_WORKSPACE.
 */
int msgl_paged_extend(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                      const void* k_cache, const void* v_cache, int64_t num_slots,
                      int64_t cache_row_stride, const int32_t* page_table,
                      int64_t page_table_stride, const int32_t* req_rows,
                      const int32_t* prefix_lens, const int32_t* extend_lens,
                      const int32_t* q_offsets, int32_t batch, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                      int32_t max_extend_len, int32_t max_kv_len, float sm_scale,
                      int32_t causal, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Bytes of (optional) workspace msgl_paged_extend uses for its work list:
 * 16 + 4 * batch * ceil(max_extend_len / (256 / (num_q_heads / num_kv_heads))),
 * or 0 when there is nothing to plan. */
size_t msgl_paged_extend_workspace_size(int32_t batch, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_extend_len, int32_t max_kv_len);

/*
 * msgl_embedding_gather — vocabulary-sharded embedding lookup ("Mini-SGLang
 * complete analysis" §4.9.3: one indexing(weights, ids, vocab_range) call
 * copies one table row per token id; §4.7.8: embed_tokens is split along the
 * vocabulary across tensor-parallel ranks and combined by masked indexing
 * plus an all-reduce).  For i < n:
 *   out[i] = weights[ids[i] - vocab_start]   if 0 <= ids[i] - vocab_start < num_rows
 *   out[i] = 0                               otherwise
 * Rows are copied bit for bit.
 *
 *   out        [n, hidden] elements, row i at i * out_row_stride
 *   weights    this shard's table, [num_rows, hidden], row r at
 *              r * weight_row_stride (strides in elements, >= hidden)
 *   ids        n token ids, int32 (MSGL_INDEX_I32) or int64 (MSGL_INDEX_I64)
 *   dtype      MSGL_DTYPE_BF16 or MSGL_DTYPE_F32 (element size 2 or 4)
 * Pointers must be aligned to their element size.  n == 0 is a no-op.
 * Enqueues on `stream`; the caller owns every buffer.
 */
int msgl_embedding_gather(void* out, int64_t out_row_stride, const void* weights,
                          int64_t num_rows, int64_t weight_row_stride, const void* ids,
                          int32_t index_dtype, int64_t n, int64_t vocab_start, int32_t hidden,
                          int32_t dtype, hipStream_t stream);

/*
 * msgl_rope_cos_sin_cache — the RoPE table shared by every layer ("Mini-SGLang
 * complete analysis" §4.5.6: one cos/sin cache of max_position x rotary_dim).
 * Row p of `cache` ([max_position, rotary_dim] fp32, caller-owned) receives
 * cos(p * theta_i) in columns [0, rotary_dim/2) and sin(p * theta_i) in
 * [rotary_dim/2, rotary_dim), theta_i = base^(-2i / rotary_dim); angle and
 * functions in double precision, rounded to fp32 once.  rotary_dim must be
 * positive and even.
 */
int msgl_rope_cos_sin_cache(float* cache, int64_t max_position, int32_t rotary_dim, double base,
                            hipStream_t stream);

/*
 * msgl_qk_norm_rope_store — the attention layer's prologue, fused ("Mini-SGLang
 * complete analysis" §4.6.7: split the merged qkv into q, k, v; RMS-normalise
 * q and k per head (Qwen3's q_norm / k_norm); rotate q and k with RoPE at the
 * batch positions; store k and v into the paged pool at out_loc).  For token t
 * and head vector x (128 dims):
 *   norm(x) = x / sqrt(mean(x^2) + eps) * w      (skipped when w is NULL)
 *   rope(x)[i]      = x[i] cos(p t_i) - x[i+64] sin(p t_i)      i < 64
 *   rope(x)[i + 64] = x[i+64] cos(p t_i) + x[i] sin(p t_i)      (rotate half)
 * with cos / sin read from `cos_sin_cache` row p = positions[t] (clamped to
 * [0, max_position)).  Outputs, rounded to bf16 once:
 *   q_out[t, h]              = rope(norm_q(q[t, h]))
 *   k_cache[out_loc[t], g]   = rope(norm_k(k[t, g]))
 *   v_cache[out_loc[t], g]   = v[t, g]                 (bit copy)
 *
 *   qkv        bf16 [n, (Hq + 2 Hkv) * 128]: q heads, then k heads, then v
 *              heads; row t at t * qkv_row_stride elements
 *   q_out      bf16 [n, Hq, 128], row t at t * q_out_row_stride; may be the
 *              qkv buffer itself (q_out = qkv, same stride) for in-place use
 *   k_cache, v_cache, num_slots, cache_row_stride   as for msgl_store_kv
 *   q_norm_weight, k_norm_weight   bf16 [128] each, or NULL
 *   positions  int32 [n];  cos_sin_cache  fp32 [max_position, 128] as built by
 *              msgl_rope_cos_sin_cache
 *   out_loc    n distinct slots, int32 or int64 (index_dtype); not checked
 * head_dim must be 128, num_q_heads a multiple of num_kv_heads; rows, norm
 * weights, the table and the pool planes 16-byte aligned, row strides (qkv,
 * q_out and the pool's) multiples of 8 elements.
 * n == 0 is a no-op.
 */
int msgl_qk_norm_rope_store(void* q_out, int64_t q_out_row_stride, void* k_cache, void* v_cache,
                            int64_t num_slots, int64_t cache_row_stride, const void* qkv,
                            int64_t qkv_row_stride, const void* q_norm_weight,
                            const void* k_norm_weight, float eps, const int32_t* positions,
                            const float* cos_sin_cache, int64_t max_position, const void* out_loc,
                            int32_t index_dtype, int64_t n, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, hipStream_t stream);

/*
 * msgl_merge_states — for each (n, h): M = max_s part_lse[s, n, h],
 *   w_s = exp(part_lse[s, n, h] - M),
 *   out[n, h] = sum_s w_s part_out[s, n, h] / sum_s w_s,
 *   lse_out[n, h] = M + ln sum_s w_s.
 * Parts with lse = -inf carry no weight; if all are -inf the output is 0 and
 * lse is -inf.
 *
 *   part_out   fp32 [num_parts, n, num_heads, head_dim] contiguous
 *   part_lse   fp32 [num_parts, n, num_heads] contiguous
 *   out        [n, num_heads, head_dim] of out_dtype (bf16 or f32)
 *   lse_out    fp32 [n, num_heads] or NULL
 *   head_dim   multiple of 4, at most 256
 */
int msgl_merge_states(void* out, float* lse_out, const float* part_out,
                      const float* part_lse, int32_t num_parts, int64_t n,
                      int32_t num_heads, int32_t head_dim, int32_t out_dtype,
                      hipStream_t stream);

/*
 * Validation alone.  msgl_validate_<call> takes the arguments of msgl_<call>
 * without the stream, runs the same host-side checks in the same order and
 * returns the status that call would return before its first HIP call:
 * MSGL_OK where the call would enqueue its kernels, else the error code, with
 * msgl_last_error() describing it.  It makes no HIP call, so it works on a
 * host without a GPU; pointers are checked for NULL and alignment only, never
 * dereferenced.
 */
int msgl_validate_store_kv(void* k_cache, void* v_cache, int64_t num_slots,
                           int64_t cache_row_stride, const void* k_new, const void* v_new,
                           int64_t new_row_stride, const void* out_loc, int32_t index_dtype,
                           int64_t n, int32_t num_kv_heads, int32_t head_dim, int32_t dtype);
int msgl_validate_paged_decode(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               const void* k_cache, const void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const int32_t* page_table,
                               int64_t page_table_stride, const int32_t* req_rows,
                               const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t max_seq_len, float sm_scale, int32_t split_tokens,
                               void* workspace, size_t workspace_bytes);
int msgl_validate_store_kv_paged_decode(
    void* out, float* lse_out, const void* q, int64_t q_row_stride, void* k_cache, void* v_cache,
    int64_t num_slots, int64_t cache_row_stride, const void* k_new, const void* v_new,
    int64_t new_row_stride, const void* out_loc, int32_t index_dtype, const int32_t* page_table,
    int64_t page_table_stride, const int32_t* req_rows, const int32_t* seq_lens, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
    int32_t max_seq_len, float sm_scale, int32_t split_tokens, void* workspace,
    size_t workspace_bytes);
int msgl_validate_paged_extend(void* out, float* lse_out, const void* q, int64_t q_row_stride,
                               const void* k_cache, const void* v_cache, int64_t num_slots,
                               int64_t cache_row_stride, const int32_t* page_table,
                               int64_t page_table_stride, const int32_t* req_rows,
                               const int32_t* prefix_lens, const int32_t* extend_lens,
                               const int32_t* q_offsets, int32_t batch, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                               int32_t max_extend_len, int32_t max_kv_len, float sm_scale,
                               int32_t causal, void* workspace, size_t workspace_bytes);
int msgl_validate_merge_states(void* out, float* lse_out, const float* part_out,
                               const float* part_lse, int32_t num_parts, int64_t n,
                               int32_t num_heads, int32_t head_dim, int32_t out_dtype);

/*
 * Graph-replayed decode step ["Mini-SGLang complete analysis" §4.6.6 (the
 * attention backend's persistent capture buffers, live data written in place
 * before replay), §5.3 (one graph per batch size of [1, 2, 4, 8, 16, 24, ...,
 * max_bs], padding to the next size with a dummy request on a sentinel page)].
 *
 * A msgl_decode_graph owns one captured HIP graph per ladder size, each
 * holding the padding of the batch and store_kv + paged_decode (balanced
 * split-KV) for that many rows of fixed-address buffers carved from caller
 * memory `buffer`.  With fused_store != 0 the step is captured as
 * msgl_store_kv_paged_decode (one launch for store + attention), which
 * needs that call's allocator contract on every replay: out_loc[r] ==
 * page_table[req_rows[r], seq_lens[r] - 1] and no request's keys include
 * another request's out_loc (the padded rows all share the sentinel slot,
 * which they write with the same zero row).  With fused_store == 0 it is
 * msgl_store_kv followed by msgl_paged_decode, for any table.  Buffers:
 *   q      bf16 [max_bs, num_q_heads, 128]     k_new, v_new  bf16 [max_bs, num_kv_heads, 128]
 *   out    bf16 [max_bs, num_q_heads, 128]     lse           fp32 [max_bs, num_q_heads]
 *   seq_lens, req_rows, out_loc  int32 [max_bs]   then the decode workspace,
 * at the byte offsets msgl_decode_graph_layout() gives (offsets[0..8] in
 * that order, offsets[9] = bytes needed; every region 256-byte aligned).
 * Per step the caller writes rows [0, batch) of q, k_new, v_new, seq_lens
 * (counting the new token), req_rows and out_loc, then calls
 * msgl_decode_graph_run(batch): rows [batch, bucket) are turned into the
 * dummy request (seq_len 1, page-table row dummy_row, out_loc
 * sentinel_slot, zero q/k/v) and the bucket's graph is replayed on `stream`.
 * Results: rows [0, batch) of out / lse.
 *
 *   page_table[dummy_row, 0] must hold sentinel_slot, a slot no request owns
 *   (the pages reserve one extra page for it); padded rows all write zeros
 *   there, and so does create (its warm-up runs fully padded batches).  The
 *   pool, the page table and the buffer must stay at their addresses while
 *   the graph lives.
 * create: validates (same rules as the two calls), warms up and captures on a
 *   private stream, synchronises it; allocates the graphs (host/runtime
 *   objects) — a set-up call.  run: sets the padding node's row range on
 *   the instantiated graph (a host-side update) and launches the graph once;
 *   no allocation, no synchronisation.  Replays on one graph must not
 *   overlap (they share the buffers and the graphs).  The padding, the step
 *   and the results follow the stream order of `stream`.
 */
typedef struct msgl_decode_graph msgl_decode_graph;

int msgl_decode_graph_layout(int32_t max_bs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, size_t* offsets /* [10] */);

int msgl_decode_graph_create(void* k_cache, void* v_cache, int64_t num_slots,
                             int64_t cache_row_stride, const int32_t* page_table,
                             int64_t page_table_stride, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size, int32_t max_bs,
                             int32_t max_seq_len, float sm_scale, int32_t dummy_row,
                             int32_t sentinel_slot, int32_t fused_store, void* buffer,
                             size_t buffer_bytes, msgl_decode_graph** out);

/* batch in [0, max_bs]; 0 enqueues nothing. */
int msgl_decode_graph_run(msgl_decode_graph* graph, int32_t batch, hipStream_t stream);

/* Captured size a batch replays (-1 if out of range). */
int32_t msgl_decode_graph_bucket(const msgl_decode_graph* graph, int32_t batch);

void msgl_decode_graph_destroy(msgl_decode_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* MSGL_H */
