// Host driver for slots.cpp under AddressSanitizer + UBSan: random operation
// streams (valid and refused allocations and frees, batches that wrap around
// the ring buffer) against a plain std::deque model of the free list, for
// both policies and pool sizes from 1 page up. Prints "<n> failures".
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <deque>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "kvslots.h"
#include "kvtier.h"

namespace kvt {
void set_error(const std::string &) {}
}

int main() {
  std::mt19937_64 rng(23);
  int failures = 0;
  auto fail = [&](const char *what, int64_t pages, int policy, int step) {
    if (failures < 10)
      printf("mismatch (%s) pages=%lld policy=%d step=%d\n", what, (long long)pages, policy, step);
    failures++;
  };
  for (int64_t P : {1, 2, 3, 5, 16, 97, 1000}) {
    for (int policy : {KV_FREE_FIFO, KV_FREE_LIFO}) {
      kv_slots_t *a = nullptr;
      if (kv_slots_create(P, policy, &a) != KV_OK) return 2;
      std::deque<int64_t> model;
      for (int64_t p = 0; p < P; p++) model.push_back(p);
      std::vector<int64_t> held, out((size_t)P + 2), snap((size_t)P);
      const int steps = P <= 16 ? 4000 : 1500;
      for (int step = 0; step < steps; step++) {
        const uint64_t r = rng() % 10;
        if (r < 4 && !held.empty()) {  // valid free of a random subset, random order
          std::shuffle(held.begin(), held.end(), rng);
          const size_t m = 1 + rng() % held.size();
          std::vector<int64_t> batch(held.end() - m, held.end());
          held.resize(held.size() - m);
          if (kv_slots_free(a, batch.data(), (int64_t)m) != KV_OK) fail("free", P, policy, step);
          if (policy == KV_FREE_FIFO)
            model.insert(model.end(), batch.begin(), batch.end());
          else
            model.insert(model.begin(), batch.begin(), batch.end());
        } else if (r < 5) {  // refused free: range, double free or a page listed twice
          std::vector<int64_t> batch;
          if (!held.empty()) batch.push_back(held[rng() % held.size()]);
          const uint64_t kind = rng() % 3;
          int want = KV_EINVAL;
          if (kind == 0) {
            batch.push_back(rng() % 2 ? -1 : P + (int64_t)(rng() % 4));
            want = KV_ERANGE;
          } else if (kind == 1 && !held.empty()) {
            batch.push_back(batch[0]);
          } else if (!model.empty()) {
            batch.push_back(model[rng() % model.size()]);
          } else {
            batch.push_back(P);
            want = KV_ERANGE;
          }
          if (kv_slots_free(a, batch.data(), (int64_t)batch.size()) != want)
            fail("refused free", P, policy, step);
        } else {  // allocation, sometimes one page too many
          int64_t k = (int64_t)(rng() % (uint64_t)(P / 2 + 2));
          if (rng() % 8 == 0) k = (int64_t)model.size() + 1;
          const int rc = kv_slots_alloc(a, k, out.data());
          if (k > (int64_t)model.size()) {
            if (rc != KV_ENOMEM) fail("enomem", P, policy, step);
          } else {
            if (rc != KV_OK) fail("alloc rc", P, policy, step);
            for (int64_t i = 0; i < k; i++) {
              if (out[(size_t)i] != model.front()) {
                fail("alloc pages", P, policy, step);
                break;
              }
              held.push_back(model.front());
              model.pop_front();
            }
          }
        }
        const int64_t n = kv_slots_snapshot(a, snap.data(), P);
        bool ok = n == (int64_t)model.size() && kv_slots_available(a) == n;
        for (int64_t i = 0; ok && i < n; i++) ok = snap[(size_t)i] == model[(size_t)i];
        if (!ok) {
          fail("free list", P, policy, step);
          break;
        }
      }
      std::set<int64_t> all(held.begin(), held.end());
      all.insert(model.begin(), model.end());
      if ((int64_t)all.size() != P || (int64_t)(held.size() + model.size()) != P)
        fail("partition", P, policy, -1);
      kv_slots_destroy(a);
    }
  }
  printf("%d failures\n", failures);
  return failures ? 1 : 0;
}
