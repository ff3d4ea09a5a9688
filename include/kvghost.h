/* kvghost.h — write-through-selective filter with a Ghost List (host only).
 *
 * The step before a D2H write-back that decides which pages it moves
 * ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.6, "Write-policy
 * semantic fix + Ghost List"; "Baidu's KVCache Overhaul", "write_through_selective
 * with Ghost List"). When pages leave the GPU pool their KV is dropped but their
 * page hashes are remembered in a bounded list; when a prefix is rebuilt, a hash
 * found in that list proves the prefix up to that page is reused, and only that
 * part is written back to the host pool with kv_backup.
 *
 * Page-boundary hash: the hash at the end of page k covers every token from the
 * root to that boundary, so it names the page's content and its position. It is
 * 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 0x100000001b3, per byte
 * xor then multiply modulo 2^64) over the token ids as 4-byte little-endian
 * signed integers. A trailing partial page has no hash.
 *
 * Ghost List: hashes in least-recently-inserted order, at most `capacity` of
 * them. Inserting a present hash makes it the most recent; inserting into a
 * full list first drops the least recent. Lookups do not change the order.
 * Every operation is O(1) per hash; an entry takes 24 bytes (the hash, two
 * 4-byte list links, and two 4-byte slots of an open-addressing index table
 * kept at most half full).
 *
 * All functions run on the host; none needs a GPU. A list may be used from
 * several threads: each call takes the list's lock.
 *
 * Status codes are those of kvtier.h (KV_OK, KV_EINVAL, KV_ENOMEM); the message
 * of the last failure on the calling thread is kv_last_error(). */
#ifndef KVGHOST_H
#define KVGHOST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_ghost kv_ghost_t; /* opaque */

/* Page-boundary hashes of one token sequence: writes n_tokens / page_size
 * hashes to out (caller-owned, that many entries). Returns the number written
 * (>= 0), or KV_EINVAL for page_size < 1, n_tokens < 0, or a null pointer
 * with n_tokens >= page_size. Cost O(n_tokens). */
int64_t kv_page_hashes(const int32_t *tokens, int64_t n_tokens, int32_t page_size,
                       uint64_t *out);

/* Creates an empty list holding at most `capacity` hashes (1 <= capacity <=
 * 2^30), all memory allocated here. KV_EINVAL for a bad capacity or null out,
 * KV_ENOMEM if the allocation fails. */
int kv_ghost_create(int64_t capacity, kv_ghost_t **out);

/* Frees the list. NULL is a no-op. */
int kv_ghost_destroy(kv_ghost_t *g);

/* Records n evicted page hashes, in order (hashes borrowed for the call).
 * KV_EINVAL for a null list, n < 0, or null hashes with n > 0. */
int kv_ghost_insert(kv_ghost_t *g, const uint64_t *hashes, int64_t n);

/* The longest proven-reuse prefix of a rebuilt sequence: scans hashes from
 * the last page back and returns k where hashes[k-1] is the first hash found
 * in the list, or 0 if none is. The caller writes back pages [0, k). Returns
 * KV_EINVAL (negative) for a null list, n < 0, or null hashes with n > 0. */
int64_t kv_ghost_reuse_prefix(kv_ghost_t *g, const uint64_t *hashes, int64_t n);

/* 1 if h is in the list, 0 if not, KV_EINVAL for a null list. */
int kv_ghost_contains(kv_ghost_t *g, uint64_t h);

/* Number of hashes held (>= 0), or KV_EINVAL for a null list. */
int64_t kv_ghost_size(kv_ghost_t *g);

/* Copies the held hashes, least recent first, into out (up to max entries);
 * returns the number copied, or KV_EINVAL. For tests and inspection. */
int64_t kv_ghost_snapshot(kv_ghost_t *g, uint64_t *out, int64_t max);

#ifdef __cplusplus
}
#endif

#endif /* KVGHOST_H */
