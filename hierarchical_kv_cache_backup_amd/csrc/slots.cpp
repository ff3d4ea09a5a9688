// slots.cpp — page allocator of the host KV pool (see include/kvslots.h).
//
// The free list is a ring buffer of num_pages page ids holding `count` live
// entries from `head`; both policies allocate from the head, FIFO frees at the
// tail and LIFO frees just before the head. One state byte per page
// (free / allocated / seen in the batch being freed) checks a free batch in
// O(batch) before anything changes.
#include <cstdint>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kvslots.h"
#include "kvtier.h"

namespace kvt {
void set_error(const std::string &msg);  // kvtier.cpp (thread-local)
}

namespace {

constexpr int64_t kMaxPages = (int64_t)1 << 40;
enum : uint8_t { kFree = 0, kAllocated = 1, kInBatch = 2 };

int fail(int code, const std::string &msg) {
  kvt::set_error(msg);
  return code;
}

}  // namespace

struct kv_slots {
  std::mutex mu;
  int64_t pages = 0;
  int32_t policy = KV_FREE_FIFO;
  std::vector<int64_t> ring;
  std::vector<uint8_t> state;
  int64_t head = 0, count = 0;

  int64_t at(int64_t k) const {  // ring position k entries after the head
    int64_t p = head + k;
    return p >= pages ? p - pages : p;
  }
};

extern "C" {

int kv_slots_create(int64_t num_pages, int32_t policy, kv_slots_t **out) {
  if (!out) return fail(KV_EINVAL, "kv_slots_create: out is null");
  *out = nullptr;
  if (num_pages < 1 || num_pages > kMaxPages)
    return fail(KV_EINVAL, "kv_slots_create: num_pages must be in [1, 2^40]");
  if (policy != KV_FREE_FIFO && policy != KV_FREE_LIFO)
    return fail(KV_EINVAL, "kv_slots_create: policy must be KV_FREE_FIFO or KV_FREE_LIFO");
  kv_slots *a = new (std::nothrow) kv_slots;
  if (!a) return fail(KV_ENOMEM, "kv_slots_create: out of memory");
  try {
    a->ring.resize((size_t)num_pages);
    a->state.assign((size_t)num_pages, kFree);
  } catch (const std::bad_alloc &) {
    delete a;
    return fail(KV_ENOMEM, "kv_slots_create: out of memory");
  }
  for (int64_t p = 0; p < num_pages; p++) a->ring[(size_t)p] = p;
  a->pages = num_pages;
  a->policy = policy;
  a->head = 0;
  a->count = num_pages;
  *out = a;
  return KV_OK;
}

int kv_slots_destroy(kv_slots_t *a) {
  delete a;
  return KV_OK;
}

int kv_slots_alloc(kv_slots_t *a, int64_t n, int64_t *out) {
  if (!a) return fail(KV_EINVAL, "kv_slots_alloc: allocator is null");
  if (n < 0) return fail(KV_EINVAL, "kv_slots_alloc: n < 0");
  if (n > 0 && !out) return fail(KV_EINVAL, "kv_slots_alloc: out is null");
  std::lock_guard<std::mutex> lock(a->mu);
  if (n > a->count)
    return fail(KV_ENOMEM, "kv_slots_alloc: " + std::to_string(n) + " pages asked, " +
                               std::to_string(a->count) + " free");
  for (int64_t k = 0; k < n; k++) {
    const int64_t p = a->ring[(size_t)a->at(k)];
    out[k] = p;
    a->state[(size_t)p] = kAllocated;
  }
  a->head = n == 0 ? a->head : a->at(n % a->pages);
  a->count -= n;
  if (a->count == 0) a->head = 0;
  return KV_OK;
}

int kv_slots_free(kv_slots_t *a, const int64_t *pages, int64_t n) {
  if (!a) return fail(KV_EINVAL, "kv_slots_free: allocator is null");
  if (n < 0) return fail(KV_EINVAL, "kv_slots_free: n < 0");
  if (n > 0 && !pages) return fail(KV_EINVAL, "kv_slots_free: pages is null");
  std::lock_guard<std::mutex> lock(a->mu);
  for (int64_t k = 0; k < n; k++)
    if (pages[k] < 0 || pages[k] >= a->pages)
      return fail(KV_ERANGE, "kv_slots_free: page " + std::to_string(pages[k]) +
                                 " outside [0, " + std::to_string(a->pages) + ")");
  int64_t bad = -1;
  for (int64_t k = 0; k < n && bad < 0; k++) {
    uint8_t &s = a->state[(size_t)pages[k]];
    if (s == kAllocated)
      s = kInBatch;
    else
      bad = k;
  }
  if (bad >= 0) {
    const int64_t p = pages[bad];
    const bool twice = a->state[(size_t)p] == kInBatch;
    for (int64_t k = 0; k < bad; k++) a->state[(size_t)pages[k]] = kAllocated;
    return fail(KV_EINVAL, "kv_slots_free: page " + std::to_string(p) +
                               (twice ? " listed twice" : " is not allocated"));
  }
  // every page of the batch was allocated, so n <= pages - count
  if (a->policy == KV_FREE_FIFO) {
    for (int64_t k = 0; k < n; k++) a->ring[(size_t)a->at(a->count + k)] = pages[k];
  } else {
    a->head = a->at(a->pages - n);  // head - n (mod pages); n <= pages
    for (int64_t k = 0; k < n; k++) a->ring[(size_t)a->at(k)] = pages[k];
  }
  for (int64_t k = 0; k < n; k++) a->state[(size_t)pages[k]] = kFree;
  a->count += n;
  return KV_OK;
}

int64_t kv_slots_available(kv_slots_t *a) {
  if (!a) return fail(KV_EINVAL, "kv_slots_available: allocator is null");
  std::lock_guard<std::mutex> lock(a->mu);
  return a->count;
}

int64_t kv_slots_snapshot(kv_slots_t *a, int64_t *out, int64_t max) {
  if (!a) return fail(KV_EINVAL, "kv_slots_snapshot: allocator is null");
  if (max < 0 || (max > 0 && !out)) return fail(KV_EINVAL, "kv_slots_snapshot: bad output");
  std::lock_guard<std::mutex> lock(a->mu);
  const int64_t m = max < a->count ? max : a->count;
  for (int64_t k = 0; k < m; k++) out[k] = a->ring[(size_t)a->at(k)];
  return m;
}

}  // extern "C"
