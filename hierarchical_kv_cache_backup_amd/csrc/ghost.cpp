// ghost.cpp — page-boundary hashes and the Ghost List (see include/kvghost.h).
//
// The list is a fixed-capacity slab of entries {hash, prev, next} threaded on a
// doubly linked recency list (head = least recent, tail = most recent) and
// indexed by an open-addressing table with linear probing. Deletion from the
// table shifts the following probe run back instead of leaving tombstones, so
// lookups stay short however long the list lives.
#include <cstdint>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kvghost.h"
#include "kvtier.h"

namespace kvt {
void set_error(const std::string &msg);  // kvtier.cpp (thread-local)
}

namespace {

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

// Table index of a key: the keys are usually FNV hashes already, but callers
// may insert any value, so the index goes through a 64-bit finalizer
// (SplitMix64's output mix).
inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

int fail(int code, const std::string &msg) {
  kvt::set_error(msg);
  return code;
}

}  // namespace

struct kv_ghost {
  std::mutex mu;
  int64_t cap = 0;
  int64_t count = 0;  // slots in use; slots [0, count) are live
  std::vector<uint64_t> key;
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1;
  std::vector<int32_t> table;  // slot index or -1
  uint64_t mask = 0;

  uint64_t home(uint64_t h) const { return mix(h) & mask; }

  int32_t find(uint64_t h, uint64_t *pos) const {
    uint64_t i = home(h);
    while (table[i] >= 0) {
      if (key[table[i]] == h) {
        if (pos) *pos = i;
        return table[i];
      }
      i = (i + 1) & mask;
    }
    if (pos) *pos = i;
    return -1;
  }

  void table_erase(uint64_t p) {
    table[p] = -1;
    uint64_t j = (p + 1) & mask;
    while (table[j] >= 0) {
      const uint64_t k = home(key[table[j]]);
      // the entry at j may fill the hole at p unless its home lies in (p, j]
      const bool home_in_range = p < j ? (k > p && k <= j) : (k > p || k <= j);
      if (!home_in_range) {
        table[p] = table[j];
        table[j] = -1;
        p = j;
      }
      j = (j + 1) & mask;
    }
  }

  void unlink(int32_t s) {
    if (prev[s] >= 0) next[prev[s]] = next[s]; else head = next[s];
    if (next[s] >= 0) prev[next[s]] = prev[s]; else tail = prev[s];
    prev[s] = next[s] = -1;
  }

  void push_tail(int32_t s) {
    prev[s] = tail;
    next[s] = -1;
    if (tail >= 0) next[tail] = s; else head = s;
    tail = s;
  }

  void insert(uint64_t h) {
    uint64_t pos = 0;
    int32_t s = find(h, &pos);
    if (s >= 0) {  // present: becomes the most recent
      if (s != tail) {
        unlink(s);
        push_tail(s);
      }
      return;
    }
    if (count == cap) {  // full: the least recent gives up its slot
      s = head;
      unlink(s);
      uint64_t vp = 0;
      (void)find(key[s], &vp);
      table_erase(vp);
      (void)find(h, &pos);  // the erase may have moved the probe run
    } else {
      s = (int32_t)count++;
    }
    key[s] = h;
    push_tail(s);
    table[pos] = s;
  }
};

extern "C" int64_t kv_page_hashes(const int32_t *tokens, int64_t n_tokens, int32_t page_size,
                                  uint64_t *out) {
  if (page_size < 1) return fail(KV_EINVAL, "page_size must be >= 1");
  if (n_tokens < 0) return fail(KV_EINVAL, "n_tokens must be >= 0");
  const int64_t pages = n_tokens / page_size;
  if (pages > 0 && (!tokens || !out)) return fail(KV_EINVAL, "null tokens or out");
  uint64_t h = kFnvOffset;
  for (int64_t k = 0; k < pages; k++) {
    const int32_t *t = tokens + k * page_size;
    for (int32_t j = 0; j < page_size; j++) {
      const uint32_t v = (uint32_t)t[j];
      for (int b = 0; b < 4; b++) {  // little-endian bytes of the token id
        h ^= (v >> (8 * b)) & 0xffu;
        h *= kFnvPrime;
      }
    }
    out[k] = h;
  }
  return pages;
}

extern "C" int kv_ghost_create(int64_t capacity, kv_ghost_t **out) {
  if (!out) return fail(KV_EINVAL, "out is null");
  *out = nullptr;
  if (capacity < 1 || capacity > (int64_t(1) << 30))
    return fail(KV_EINVAL, "capacity must be in [1, 2^30]");
  kv_ghost *g = new (std::nothrow) kv_ghost;
  if (!g) return fail(KV_ENOMEM, "allocating the Ghost List");
  try {
    g->cap = capacity;
    g->key.assign((size_t)capacity, 0);
    g->prev.assign((size_t)capacity, -1);
    g->next.assign((size_t)capacity, -1);
    uint64_t tsize = 2;
    while (tsize < 2 * (uint64_t)capacity) tsize <<= 1;
    g->table.assign(tsize, -1);
    g->mask = tsize - 1;
  } catch (const std::bad_alloc &) {
    delete g;
    return fail(KV_ENOMEM, "allocating the Ghost List");
  }
  *out = g;
  return KV_OK;
}

extern "C" int kv_ghost_destroy(kv_ghost_t *g) {
  delete g;
  return KV_OK;
}

extern "C" int kv_ghost_insert(kv_ghost_t *g, const uint64_t *hashes, int64_t n) {
  if (!g) return fail(KV_EINVAL, "null list");
  if (n < 0 || (n > 0 && !hashes)) return fail(KV_EINVAL, "bad hashes or n");
  std::lock_guard<std::mutex> lock(g->mu);
  for (int64_t i = 0; i < n; i++) g->insert(hashes[i]);
  return KV_OK;
}

extern "C" int64_t kv_ghost_reuse_prefix(kv_ghost_t *g, const uint64_t *hashes, int64_t n) {
  if (!g) return fail(KV_EINVAL, "null list");
  if (n < 0 || (n > 0 && !hashes)) return fail(KV_EINVAL, "bad hashes or n");
  std::lock_guard<std::mutex> lock(g->mu);
  for (int64_t k = n - 1; k >= 0; k--)
    if (g->find(hashes[k], nullptr) >= 0) return k + 1;
  return 0;
}

extern "C" int kv_ghost_contains(kv_ghost_t *g, uint64_t h) {
  if (!g) return fail(KV_EINVAL, "null list");
  std::lock_guard<std::mutex> lock(g->mu);
  return g->find(h, nullptr) >= 0 ? 1 : 0;
}

extern "C" int64_t kv_ghost_size(kv_ghost_t *g) {
  if (!g) return fail(KV_EINVAL, "null list");
  std::lock_guard<std::mutex> lock(g->mu);
  return g->count;
}

extern "C" int64_t kv_ghost_snapshot(kv_ghost_t *g, uint64_t *out, int64_t max) {
  if (!g) return fail(KV_EINVAL, "null list");
  if (max < 0 || (max > 0 && !out)) return fail(KV_EINVAL, "bad out or max");
  std::lock_guard<std::mutex> lock(g->mu);
  int64_t k = 0;
  for (int32_t s = g->head; s >= 0 && k < max; s = g->next[s]) out[k++] = g->key[s];
  return k;
}
