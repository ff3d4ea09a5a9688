/* kvslots.h — page allocator of the host KV pool, FIFO or LIFO free list (host only).
 *
 * The host pool is handed out in whole pages (page_size token slots each); a
 * write-back first takes free pages here, then moves its KV into their slots
 * with kv_backup, and evicting a cached prefix gives its pages back. The
 * allocator decides WHICH host pages a write-back touches, not whether it
 * happens: the free-list order is a locality choice with no effect on hit rate
 * or eviction ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.4,
 * "LIFO free list"; "Baidu's KVCache Overhaul", "LIFO slot allocation").
 *
 *   KV_FREE_FIFO  pages freed go to the tail of the free list; allocations take
 *                 from the head. Under churn the allocator walks through the
 *                 whole pool before it hands back a page freed earlier.
 *   KV_FREE_LIFO  pages freed go to the head of the free list; allocations take
 *                 from the head. The pages freed most recently are handed out
 *                 first, so churn keeps reusing a small set of hot pages.
 *
 * Free list and order (where the pages leave it open): the list starts as pages
 * 0, 1, ..., num_pages-1. kv_slots_alloc(k) removes and returns the first k
 * entries of the list, in list order. kv_slots_free(pages) inserts the batch,
 * keeping its order, at the tail (FIFO) or at the head (LIFO): after a LIFO
 * free of pages {a, b, c}, the next allocation of 3 pages returns a, b, c.
 *
 * Pages, not token slots: page p covers host slots [p*page_size,
 * (p+1)*page_size) of the pool kv_backup / kv_load address.
 *
 * Every call is O(pages in the call) except create (O(num_pages)). A handle may
 * be used from several threads: each call takes the allocator's lock.
 *
 * Status codes are those of kvtier.h; kv_last_error() names the failure on the
 * calling thread. A failing call changes nothing. */
#ifndef KVSLOTS_H
#define KVSLOTS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_slots kv_slots_t; /* opaque */

typedef enum { KV_FREE_FIFO = 0, KV_FREE_LIFO = 1 } kv_free_policy_t;

/* Creates an allocator over pages [0, num_pages), all free, with the given
 * policy (a kv_free_policy_t value). 1 <= num_pages <= 2^40. KV_EINVAL for a
 * bad size or policy or a null out, KV_ENOMEM if its memory (9 bytes per page)
 * cannot be allocated. */
int kv_slots_create(int64_t num_pages, int32_t policy, kv_slots_t **out);

/* Frees the allocator. NULL is a no-op. */
int kv_slots_destroy(kv_slots_t *a);

/* Takes n pages off the head of the free list and writes their ids to out
 * (caller-owned, n entries), in list order. KV_ENOMEM if fewer than n pages
 * are free (nothing is taken), KV_EINVAL for a null allocator, n < 0, or a null
 * out with n > 0. n == 0 is a successful no-op. */
int kv_slots_alloc(kv_slots_t *a, int64_t n, int64_t *out);

/* Returns n pages to the free list (pages borrowed for the call), at the tail
 * (FIFO) or the head (LIFO), in the given order. KV_ERANGE for a page outside
 * [0, num_pages); KV_EINVAL for a page that is not allocated (a double free),
 * a page listed twice, a null allocator, n < 0, or null pages with n > 0. The
 * whole batch is checked before anything changes. */
int kv_slots_free(kv_slots_t *a, const int64_t *pages, int64_t n);

/* Number of free pages (>= 0), or KV_EINVAL for a null allocator. */
int64_t kv_slots_available(kv_slots_t *a);

/* Copies the free list, head first, into out (up to max entries); returns the
 * number copied, or KV_EINVAL. For tests and inspection. */
int64_t kv_slots_snapshot(kv_slots_t *a, int64_t *out, int64_t max);

#ifdef __cplusplus
}
#endif

#endif /* KVSLOTS_H */
