// Host driver for ghost.cpp under AddressSanitizer + UBSan: random operation
// streams against a plain std::list model of the least-recently-inserted
// order, with small tables (many evictions and probe-run shifts) and large
// ones. Prints "<n> failures".
#include <cstdint>
#include <cstdio>
#include <list>
#include <random>
#include <string>
#include <vector>

#include "kvghost.h"
#include "kvtier.h"

namespace kvt {
void set_error(const std::string &) {}
}

int main() {
  std::mt19937_64 rng(11);
  int failures = 0;
  const int64_t caps[] = {1, 2, 3, 7, 16, 100, 4096};
  for (int64_t cap : caps) {
    for (uint64_t keys : {uint64_t(3), uint64_t(50), uint64_t(5000), ~uint64_t(0)}) {
      kv_ghost_t *g = nullptr;
      if (kv_ghost_create(cap, &g) != KV_OK) return 2;
      std::list<uint64_t> model;
      std::vector<uint64_t> batch, snap((size_t)cap);
      const int steps = cap <= 16 ? 3000 : 300;
      const uint64_t max_batch = cap <= 16 ? uint64_t(2 * cap + 3) : uint64_t(40);
      for (int step = 0; step < steps; step++) {
        batch.resize(rng() % max_batch);
        for (auto &h : batch) h = keys == ~uint64_t(0) ? rng() : rng() % keys;
        kv_ghost_insert(g, batch.data(), (int64_t)batch.size());
        for (uint64_t h : batch) {
          model.remove(h);
          if ((int64_t)model.size() == cap) model.pop_front();
          model.push_back(h);
        }
        if (step % 7 == 0 || cap <= 16) {
          const int64_t k = kv_ghost_snapshot(g, snap.data(), cap);
          bool ok = k == (int64_t)model.size() && kv_ghost_size(g) == k;
          int64_t i = 0;
          for (auto it = model.begin(); ok && it != model.end(); ++it, ++i) ok = snap[i] == *it;
          if (!ok) {
            if (failures < 5) printf("mismatch cap=%lld keys=%llu step=%d\n", (long long)cap,
                                     (unsigned long long)keys, step);
            failures++;
          }
          const uint64_t q = keys == ~uint64_t(0) ? (model.empty() ? rng() : model.front()) : rng() % keys;
          bool in = false;
          for (uint64_t h : model) in |= h == q;
          if (kv_ghost_contains(g, q) != (in ? 1 : 0)) failures++;
        }
      }
      kv_ghost_destroy(g);
    }
  }
  std::vector<int32_t> tok(1000);
  for (auto &t : tok) t = (int32_t)rng();
  std::vector<uint64_t> out(1000);
  if (kv_page_hashes(tok.data(), 1000, 7, out.data()) != 142) failures++;
  printf("%d failures\n", failures);
  return failures ? 1 : 0;
}
