// Host driver for slots.cpp and ghost.cpp under ThreadSanitizer: several
// threads call one page allocator and one Ghost List at once, as a backup
// thread and a load thread (and a scheduler) would. The allocator must never
// hand one page to two holders, and must end with every page free; the Ghost
// List must stay within its capacity and answer for what was inserted last.
// Prints "<n> failures"; ThreadSanitizer reports any data race on its own.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "kvghost.h"
#include "kvslots.h"
#include "kvtier.h"

namespace kvt {
thread_local std::string g_err_check;
void set_error(const std::string &msg) { g_err_check = msg; }
}  // namespace kvt

namespace {

std::atomic<int> failures{0};

void fail(const char *what, long long a, long long b) {
  if (failures.fetch_add(1) < 10) printf("failure: %s (%lld, %lld)\n", what, a, b);
}

// Each thread allocates batches, claims every page it got in a shared owner
// table (a page already claimed by someone else is a double hand-out), then
// releases its claims and frees the batch, in a shuffled order.
void allocator_worker(kv_slots_t *a, std::vector<std::atomic<int>> *owner, int id, int rounds) {
  std::mt19937_64 rng(1000 + id);
  std::vector<int64_t> got(64);
  for (int r = 0; r < rounds; r++) {
    const int64_t n = 1 + (int64_t)(rng() % 64);
    const int rc = kv_slots_alloc(a, n, got.data());
    if (rc == KV_ENOMEM) continue;  // the others hold the pages right now
    if (rc != KV_OK) {
      fail("alloc", rc, n);
      continue;
    }
    for (int64_t i = 0; i < n; i++) {
      int expect = -1;
      if (!(*owner)[(size_t)got[(size_t)i]].compare_exchange_strong(expect, id))
        fail("page handed out twice", got[(size_t)i], expect);
    }
    for (int64_t i = n - 1; i > 0; i--) std::swap(got[(size_t)i], got[(size_t)(rng() % (i + 1))]);
    for (int64_t i = 0; i < n; i++) (*owner)[(size_t)got[(size_t)i]].store(-1);
    if (kv_slots_free(a, got.data(), n) != KV_OK) fail("free", id, n);
  }
}

void ghost_worker(kv_ghost_t *g, int64_t capacity, int id, int rounds) {
  std::mt19937_64 rng(2000 + id);
  std::vector<uint64_t> h(64);
  for (int r = 0; r < rounds; r++) {
    const int64_t n = 1 + (int64_t)(rng() % 64);
    for (int64_t i = 0; i < n; i++) h[(size_t)i] = ((uint64_t)id << 56) | (rng() >> 8);
    if (kv_ghost_insert(g, h.data(), n) != KV_OK) fail("insert", id, n);
    const int64_t k = kv_ghost_reuse_prefix(g, h.data(), n);
    if (k < 0 || k > n) fail("reuse prefix out of range", k, n);
    const int64_t sz = kv_ghost_size(g);
    if (sz < 0 || sz > capacity) fail("size out of range", sz, capacity);
    if (kv_ghost_contains(g, h[0]) < 0) fail("contains", id, r);
  }
}

}  // namespace

int main() {
  const int kThreads = 4;
  for (int64_t pages : {64, 200, 4096}) {
    for (int policy : {KV_FREE_FIFO, KV_FREE_LIFO}) {
      kv_slots_t *a = nullptr;
      if (kv_slots_create(pages, policy, &a) != KV_OK) return 2;
      std::vector<std::atomic<int>> owner((size_t)pages);
      for (auto &o : owner) o.store(-1);
      std::vector<std::thread> th;
      for (int t = 0; t < kThreads; t++) th.emplace_back(allocator_worker, a, &owner, t, 3000);
      for (auto &x : th) x.join();
      if (kv_slots_available(a) != pages) fail("pages lost", kv_slots_available(a), pages);
      kv_slots_destroy(a);
    }
  }
  for (int64_t capacity : {16, 1000, 100000}) {
    kv_ghost_t *g = nullptr;
    if (kv_ghost_create(capacity, &g) != KV_OK) return 2;
    std::vector<std::thread> th;
    for (int t = 0; t < kThreads; t++) th.emplace_back(ghost_worker, g, capacity, t, 3000);
    for (auto &x : th) x.join();
    // the list keeps the most recent hashes: a batch inserted alone is there
    std::vector<uint64_t> last(8);
    for (size_t i = 0; i < last.size(); i++) last[i] = 0xabcdef00ull + i;
    kv_ghost_insert(g, last.data(), (int64_t)last.size());
    for (uint64_t v : last)
      if ((int64_t)last.size() <= capacity && kv_ghost_contains(g, v) != 1)
        fail("latest hash missing", (long long)v, capacity);
    kv_ghost_destroy(g);
  }
  printf("%d failures\n", failures.load());
  return failures.load() == 0 ? 0 : 1;
}
