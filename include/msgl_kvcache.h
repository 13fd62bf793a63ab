/*
 * msgl_kvcache.h — C ABI of the host-side KV cache manager: the page
 * allocator and radix prefix cache that produce the page-table rows the
 * attention calls of msgl.h consume.
 *
 * Source: "Mini-SGLang complete analysis" §4.4 (KV cache pool and radix
 * prefix cache): §4.4.4 radix tree nodes (token run, slot run, reference
 * count, LRU time), §4.4.5 page-aligned prefix matching with node splits and
 * the first-mismatch key compare, §4.4.6 locking and LRU eviction of unlocked
 * leaves, §4.4.7 allocate_paged / cache_req; "Mini-sglang deep-analysis
 * report", KV cache management (protected / evictable / free).
 *
 * Host memory only; no HIP call.  One manager is NOT thread-safe.
 *
 * Model
 * -----
 * - The pool has num_slots token slots in pages of page_size consecutive
 *   slots; the free list holds whole pages, first in first out.
 * - The manager owns a host page table int32 [max_rows, max_len] (row-major,
 *   row stride max_len): entry (row, j) is the slot of token j of the request
 *   holding the row (the layout msgl_paged_decode / msgl_paged_extend read;
 *   the caller copies rows to the device).
 * - Token ids are int32.  A "handle" is a node of the radix tree, named by an
 *   int64 id; 0 is the root (empty prefix).  A handle stays valid while it is
 *   locked (an unlocked node may be evicted or, when split, keep only the
 *   lower part of its run; the id then still names the same end position).
 *   msgl_kvc_handle_len() gives the prefix length a handle stands for.
 * - Lengths in the tree are whole pages: a match, an insert and a handle
 *   length are multiples of page_size.
 *
 * Return value: MSGL_KVC_OK (0) or a negative status; nothing is changed by a
 * call that returns MSGL_KVC_ERR_ARG or MSGL_KVC_ERR_STATE.
 */
#ifndef MSGL_KVCACHE_H
#define MSGL_KVCACHE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum msgl_kvc_status {
  MSGL_KVC_OK = 0,
  MSGL_KVC_ERR_ARG = -1,     /* bad pointer, size, row or handle                 */
  MSGL_KVC_ERR_FULL = -2,    /* not enough free pages (after eviction) or rows   */
  MSGL_KVC_ERR_STATE = -3,   /* call out of order (e.g. unlock of an unlocked path) */
  MSGL_KVC_ERR_NOMEM = -4    /* host allocation failed                           */
};

typedef struct msgl_kv_cache msgl_kv_cache;

/* New manager: num_slots slots (num_slots / page_size whole pages are used),
 * max_rows page-table rows of max_len entries (a multiple of page_size).
 * *out receives the manager; destroy it with msgl_kvc_destroy. */
int msgl_kvc_create(int64_t num_slots, int32_t page_size, int32_t max_rows, int32_t max_len,
                    msgl_kv_cache** out);
void msgl_kvc_destroy(msgl_kv_cache* kvc);

/* Host page table [max_rows, max_len], owned by the manager, valid until
 * msgl_kvc_destroy. */
const int32_t* msgl_kvc_page_table(const msgl_kv_cache* kvc);

/* Take a free page-table row (FIFO) / give one back (its pages must have been
 * released: msgl_kvc_release or a finished msgl_kvc_cache_req). */
int msgl_kvc_alloc_row(msgl_kv_cache* kvc, int32_t* row);
int msgl_kvc_free_row(msgl_kv_cache* kvc, int32_t row);

/* Longest page-aligned prefix of ids[0, n) held by the tree (§4.4.5): nodes
 * matched in full get a new LRU time, a node matched in part is split.
 * *cached_len = the prefix length, *handle = the node ending it (0: none).
 * With row >= 0 (a row holding no pages yet; n <= max_len) the prefix's
 * slots are written to page_table[row, 0 .. *cached_len).  Does not lock. */
int msgl_kvc_match(msgl_kv_cache* kvc, const int32_t* ids, int64_t n, int32_t row,
                   int64_t* cached_len, int64_t* handle);

/* delta = +1: lock the path root -> handle (its tokens move from evictable
 * to protected); delta = -1: unlock it (MSGL_KVC_ERR_STATE if not locked). */
int msgl_kvc_lock(msgl_kv_cache* kvc, int64_t handle, int32_t delta);

/* allocate_paged (§4.4.7): request i (row rows[i], cached_lens[i] tokens
 * already in place, device_lens[i] after this step) gets
 * ceil(device/P) - ceil(cached/P) new pages, written to
 * page_table[row, ceil(cached/P)*P .. ceil(device/P)*P).  When the free list
 * is short, unlocked leaves are evicted first (LRU).  All or nothing:
 * MSGL_KVC_ERR_FULL leaves every row as it was (evictions already made stay
 * made). */
int msgl_kvc_allocate(msgl_kv_cache* kvc, int32_t n, const int32_t* rows,
                      const int64_t* cached_lens, const int64_t* device_lens);

/* cache_req (§4.4.7): insert ids[0, floor(cached_len/P)*P) with the row's
 * slots; unlock old_handle (the handle the request held, 0 for none); free
 * the request's pages that the tree already held (another request inserted
 * them first) and point the row at the tree's pages; then either lock the
 * new path (finished == 0) or free the row's pages past it (finished != 0,
 * the row then holds no pages).  *new_handle / *new_len: the new handle and
 * its length. */
int msgl_kvc_cache_req(msgl_kv_cache* kvc, int32_t row, const int32_t* ids, int64_t cached_len,
                       int64_t old_handle, int32_t finished, int64_t* new_handle,
                       int64_t* new_len);

/* Drop a request without caching it: unlock handle, free the row's pages
 * past the handle's length. */
int msgl_kvc_release(msgl_kv_cache* kvc, int32_t row, int64_t handle);

/* Evict unlocked leaves, oldest first, until `pages` pages were freed or
 * none is left; *freed (may be NULL) = pages freed. */
int msgl_kvc_evict(msgl_kv_cache* kvc, int64_t pages, int64_t* freed);

/* out[0..n) of: free pages, evictable tokens, protected tokens, tree nodes
 * (root excluded), free rows, logical clock. */
int msgl_kvc_stats(const msgl_kv_cache* kvc, int64_t* out, int32_t n);

/* Free pages in order (first slot of each); copies up to cap, returns the
 * count (-1 on a NULL manager). */
int64_t msgl_kvc_free_list(const msgl_kv_cache* kvc, int32_t* out, int64_t cap);

/* End of the slots a row holds ([0, len) of its page-table row; -1: bad row). */
int64_t msgl_kvc_row_len(const msgl_kv_cache* kvc, int32_t row);

/* Prefix length a handle stands for (-1: not a live node). */
int64_t msgl_kvc_handle_len(const msgl_kv_cache* kvc, int64_t handle);

/* Length of the common prefix of a[0, na) and b[0, nb): the first position
 * where they differ (§4.4.5's key compare). */
int64_t msgl_compare_key(const int32_t* a, int64_t na, const int32_t* b, int64_t nb);

#ifdef __cplusplus
}
#endif

#endif /* MSGL_KVCACHE_H */
