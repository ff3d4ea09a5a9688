// plan.cpp — host-side planner: geometry and request validation, the host
// address map, and the run-length coalescer feeding the copy-engine path.
// No HIP dependency: it is built into libkvtier.so and, for sanitizer tests,
// on its own with the host compiler.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <limits>
#include <new>
#include <utility>

namespace kvt {

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *out = a * b;
  return true;
}

std::string fmt(const char *f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

}  // namespace

int make_geom(const kv_geometry_t *in, Geom *g, std::string *why) {
  if (!in) {
    *why = "geometry is null";
    return KV_EINVAL;
  }
  if (in->num_layers < 1 || in->num_components < 1 || in->page_size < 1) {
    *why = "num_layers, num_components and page_size must be >= 1";
    return KV_EINVAL;
  }
  if (in->row_bytes < 16 || in->row_bytes % 16 != 0) {
    *why = fmt("row_bytes (%lld) must be a positive multiple of 16", in->row_bytes);
    return KV_EINVAL;
  }
  if (in->row_bytes > kRowBytesLimit) {
    *why = fmt("row_bytes (%lld) exceeds the library's limit of 2^30", in->row_bytes);
    return KV_EINVAL;
  }
  if (in->device_slots < 1 || in->host_slots < 1) {
    *why = "device_slots and host_slots must be >= 1";
    return KV_EINVAL;
  }
  if (in->host_slots % in->page_size != 0) {
    *why = fmt("host_slots (%lld) must be a multiple of page_size (%lld)", in->host_slots,
               in->page_size);
    return KV_EINVAL;
  }
  if (in->host_layout != KV_LAYER_FIRST && in->host_layout != KV_PAGE_FIRST &&
      in->host_layout != KV_PAGE_FIRST_DIRECT) {
    *why = fmt("unknown host_layout %lld", in->host_layout);
    return KV_EINVAL;
  }
  int64_t lc, rows, bytes, dev_bytes;
  if (!mul_ok(in->num_layers, in->num_components, &lc) || !mul_ok(lc, in->host_slots, &rows) ||
      !mul_ok(rows, in->row_bytes, &bytes) || !mul_ok(in->device_slots, in->row_bytes, &dev_bytes)) {
    *why = "pool size overflows int64";
    return KV_EINVAL;
  }
  g->L = in->num_layers;
  g->C = in->num_components;
  g->R = in->row_bytes;
  g->S_dev = in->device_slots;
  g->S_host = in->host_slots;
  g->ps = in->page_size;
  g->layout = in->host_layout;
  g->lc_stride = (g->layout == KV_LAYER_FIRST) ? g->S_host
                 : (g->layout == KV_PAGE_FIRST) ? 1
                                                : g->ps;
  return KV_OK;
}

// First position whose slot appeared earlier in dst[0, n) (-1: none), slots in
// [0, slots). KV_ENOMEM if the check's memory cannot be had. Without
// may_allocate only a stamp table already covering the slots can be used, else
// KV_EINVAL.
static int first_repeat(const int64_t *dst, int64_t n, int64_t slots, UniqueScratch *scratch,
                        int64_t *dup, std::string *why, bool may_allocate) {
  *dup = -1;
  const bool table = (int64_t)scratch->stamp.size() >= slots;
  if (!table && !may_allocate) {
    *why = "the pool's uniqueness table does not cover its destination slots (more than "
           "2^24 and no earlier call sized it), so the check cannot run without allocating";
    return KV_EINVAL;
  }
  try {
    if (table || slots <= std::max<int64_t>(kStampSlotsMin, 4 * n)) {
      // one stamp per slot, kept between calls; a generation counter instead
      // of clearing
      if (!table) scratch->stamp.assign(slots, 0);
      if (++scratch->gen == 0) {  // wrapped: clear once every 2^32 calls
        std::fill(scratch->stamp.begin(), scratch->stamp.end(), 0u);
        scratch->gen = 1;
      }
      const uint32_t gen = scratch->gen;
      uint32_t *st = scratch->stamp.data();
      for (int64_t i = 0; i < n && *dup < 0; i++) {
        if (st[dst[i]] == gen) *dup = i;
        st[dst[i]] = gen;
      }
    } else {
      // far more slots than positions: sort (slot, position) pairs instead of
      // holding a stamp per slot
      std::vector<std::pair<int64_t, int64_t>> v((size_t)n);
      for (int64_t i = 0; i < n; i++) v[(size_t)i] = {dst[i], i};
      std::sort(v.begin(), v.end());
      for (size_t k = 1; k < v.size(); k++)
        if (v[k].first == v[k - 1].first && (*dup < 0 || v[k].second < *dup)) *dup = v[k].second;
    }
  } catch (const std::bad_alloc &) {
    *why = "out of memory in the destination uniqueness check";
    return KV_ENOMEM;
  }
  return KV_OK;
}

int validate(const Geom &g, int direction, const int64_t *dev_idx, const int64_t *host_idx,
             int64_t n, int32_t l0, int32_t l1, bool check_unique, UniqueScratch *scratch,
             std::string *why, bool may_allocate) {
  if (direction != 0 && direction != 1) {
    *why = "direction must be 0 (backup) or 1 (load)";
    return KV_EINVAL;
  }
  if (n < 0) {
    *why = fmt("n (%lld) must be >= 0", n);
    return KV_EINVAL;
  }
  if (n > 0 && (!dev_idx || !host_idx)) {
    *why = "index array is null";
    return KV_EINVAL;
  }
  if (l0 < 0 || l0 > l1 || l1 > g.L) {
    *why = fmt("layer range [%lld, %lld) is not inside [0, %lld]", l0, l1, g.L);
    return KV_EINVAL;
  }
  for (int64_t i = 0; i < n; i++) {
    if ((uint64_t)dev_idx[i] >= (uint64_t)g.S_dev) {
      *why = fmt("dev_idx[%lld] = %lld is outside [0, %lld)", i, dev_idx[i], g.S_dev);
      return KV_ERANGE;
    }
    if ((uint64_t)host_idx[i] >= (uint64_t)g.S_host) {
      *why = fmt("host_idx[%lld] = %lld is outside [0, %lld)", i, host_idx[i], g.S_host);
      return KV_ERANGE;
    }
  }
  if (check_unique && n > 1) {
    const int64_t *dst = direction == 0 ? host_idx : dev_idx;
    int64_t dup = -1;
    const int rc = first_repeat(dst, n, direction == 0 ? g.S_host : g.S_dev, scratch, &dup, why,
                                may_allocate);
    if (rc) return rc;
    if (dup >= 0) {
      *why = fmt(direction == 0 ? "host slot %lld is a destination twice (position %lld)"
                                : "device slot %lld is a destination twice (position %lld)",
                 dst[dup], dup);
      return KV_EDUP;
    }
  }
  return KV_OK;
}

int validate_stage(const Geom &g, int direction, const int64_t *dev_idx, int64_t n, int32_t l0,
                   int32_t l1, bool check_unique, UniqueScratch *scratch, std::string *why) {
  if (direction != 0 && direction != 1) {
    *why = "direction must be 0 (pack) or 1 (unpack)";
    return KV_EINVAL;
  }
  if (n < 0) {
    *why = fmt("n (%lld) must be >= 0", n);
    return KV_EINVAL;
  }
  if (n > 0 && !dev_idx) {
    *why = "index array is null";
    return KV_EINVAL;
  }
  if (l0 < 0 || l0 > l1 || l1 > g.L) {
    *why = fmt("layer range [%lld, %lld) is not inside [0, %lld]", l0, l1, g.L);
    return KV_EINVAL;
  }
  for (int64_t i = 0; i < n; i++)
    if ((uint64_t)dev_idx[i] >= (uint64_t)g.S_dev) {
      *why = fmt("dev_idx[%lld] = %lld is outside [0, %lld)", i, dev_idx[i], g.S_dev);
      return KV_ERANGE;
    }
  if (check_unique && direction == 1 && n > 1) {
    int64_t dup = -1;
    const int rc = first_repeat(dev_idx, n, g.S_dev, scratch, &dup, why, true);
    if (rc) return rc;
    if (dup >= 0) {
      *why = fmt("device slot %lld is a destination twice (position %lld)", dev_idx[dup], dup);
      return KV_EDUP;
    }
  }
  return KV_OK;
}

void build_runs(const Geom &g, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                std::vector<Run> *runs) {
  runs->clear();
  if (n <= 0) return;
  int64_t start = 0;
  int64_t prev_key = host_key(g, host_idx[0]);
  for (int64_t i = 1; i < n; i++) {
    const int64_t key = host_key(g, host_idx[i]);
    if (!(dev_idx[i] == dev_idx[i - 1] + 1 && key == prev_key + 1)) {
      runs->push_back({start, i - start});
      start = i;
    }
    prev_key = key;
  }
  runs->push_back({start, n - start});
}

void build_copies(const Geom &g, const std::vector<Run> &runs, const int64_t *dev_idx,
                  const int64_t *host_idx, std::vector<Copy> *copies) {
  copies->clear();
  for (const Run &r : runs) {
    const int64_t d = dev_idx[r.i0];
    const int64_t k = host_key(g, host_idx[r.i0]);
    if (!copies->empty()) {
      Copy &c = copies->back();
      if (c.len == r.len) {
        const int64_t dp = d - (c.dev0 + (c.lines - 1) * c.dev_pitch);
        const int64_t kp = k - (c.key0 + (c.lines - 1) * c.key_pitch);
        if (c.lines == 1) {
          if (dp >= r.len && kp >= r.len) {
            c.dev_pitch = dp;
            c.key_pitch = kp;
            c.lines = 2;
            continue;
          }
        } else if (dp == c.dev_pitch && kp == c.key_pitch) {
          c.lines++;
          continue;
        }
      }
    }
    copies->push_back({d, k, r.len, 1, 0, 0});
  }
}

void host_runs(const Geom &g, const int64_t *host_idx, int64_t n, std::vector<int64_t> *start) {
  start->clear();
  if (n <= 0) return;
  start->push_back(0);
  for (int64_t i = 1; i < n; i++)
    if (host_key(g, host_idx[i]) != host_key(g, host_idx[i - 1]) + 1) start->push_back(i);
  start->push_back(n);
}

void build_extents(const Geom &g, const int64_t *host_idx, int64_t n,
                   const std::vector<int64_t> &run_start, int32_t la, int32_t lb,
                   std::vector<Extent> *out) {
  out->clear();
  if (n <= 0 || lb <= la) return;
  const int64_t nlc = (int64_t)(lb - la) * g.C;
  const int64_t lc0 = (int64_t)la * g.C;
  const int64_t G = g.layout == KV_LAYER_FIRST ? n : g.layout == KV_PAGE_FIRST ? 1 : g.ps;
  auto append = [out](int64_t walk0, int64_t host0, int64_t rows) {
    if (!out->empty()) {
      Extent &e = out->back();
      if (e.walk0 + e.rows == walk0 && e.host0 + e.rows == host0) {
        e.rows += rows;
        return;
      }
    }
    out->push_back({walk0, host0, rows});
  };
  if (g.lc_stride == 1 && G == 1) {
    // page_first: a position's rows for all pairs are consecutive host rows
    for (int64_t i = 0; i < n; i++) append(i * nlc, host_key(g, host_idx[i]) + lc0, nlc);
    return;
  }
  size_t first_run = 0;  // first run that reaches into the current group
  for (int64_t g0 = 0; g0 < n; g0 += G) {
    const int64_t gsz = std::min(G, n - g0);
    const int64_t g1 = g0 + gsz;
    const int64_t walk_base = g0 * nlc;  // every earlier group is full: G * nlc rows each
    while (run_start[first_run + 1] <= g0) first_run++;
    for (int64_t lc = 0; lc < nlc; lc++) {
      for (size_t k = first_run; run_start[k] < g1; k++) {
        const int64_t i0 = std::max(run_start[k], g0);
        const int64_t i1 = std::min(run_start[k + 1], g1);
        append(walk_base + lc * gsz + (i0 - g0), (lc0 + lc) * g.lc_stride + host_key(g, host_idx[i0]),
               i1 - i0);
      }
    }
  }
}

void build_extents(const Geom &g, const int64_t *host_idx, int64_t n, int32_t la, int32_t lb,
                   std::vector<Extent> *out) {
  std::vector<int64_t> run_start;
  host_runs(g, host_idx, n, &run_start);
  build_extents(g, host_idx, n, run_start, la, lb, out);
}

void chunk_plan(int64_t walk_rows, int64_t chunk_rows, bool ramp_first, bool ramp_last,
                std::vector<int64_t> *out) {
  out->clear();
  int64_t len = (ramp_first || ramp_last) ? std::max<int64_t>(1, chunk_rows / kRampFirst)
                                          : chunk_rows;
  for (int64_t r = 0; r < walk_rows;) {
    const int64_t take = std::min(len, walk_rows - r);
    out->push_back(take);
    r += take;
    len = std::min(chunk_rows, len * kRampGrowth);
  }
  if (ramp_last && !ramp_first) std::reverse(out->begin(), out->end());
}

}  // namespace kvt

// ---- C ABI: planner entry points --------------------------------------------

namespace kvt {
void set_error(const std::string &msg);  // defined in kvtier.cpp (thread-local)
}

using namespace kvt;

extern "C" int kv_geometry_check(const kv_geometry_t *geom) {
  Geom g;
  std::string why;
  int rc = make_geom(geom, &g, &why);
  if (rc) set_error(why);
  return rc;
}

extern "C" int64_t kv_host_row(const kv_geometry_t *geom, int32_t layer, int32_t comp,
                               int64_t host_slot) {
  Geom g;
  std::string why;
  int rc = make_geom(geom, &g, &why);
  if (rc) {
    set_error(why);
    return rc;
  }
  if (layer < 0 || layer >= g.L || comp < 0 || comp >= g.C || host_slot < 0 ||
      host_slot >= g.S_host) {
    set_error("kv_host_row: argument out of range");
    return KV_ERANGE;
  }
  return host_row(g, layer, comp, host_slot);
}

extern "C" int kv_validate(const kv_geometry_t *geom, int32_t direction, const int64_t *dev_idx,
                           const int64_t *host_idx, int64_t n, int32_t layer_begin,
                           int32_t layer_end, int32_t check_unique) {
  Geom g;
  std::string why;
  int rc = make_geom(geom, &g, &why);
  if (!rc) {
    UniqueScratch scratch;
    rc = validate(g, direction, dev_idx, host_idx, n, layer_begin, layer_end, check_unique != 0,
                  &scratch, &why);
  }
  if (rc) set_error(why);
  return rc;
}

static int count_common(const kv_geometry_t *geom, const int64_t *dev_idx, const int64_t *host_idx,
                        int64_t n, int32_t l0, int32_t l1, int64_t *out, bool merge2d) {
  Geom g;
  std::string why;
  int rc = make_geom(geom, &g, &why);
  if (!rc) rc = validate(g, 0, dev_idx, host_idx, n, l0, l1, false, nullptr, &why);
  if (!rc && !out) {
    why = "out is null";
    rc = KV_EINVAL;
  }
  if (rc) {
    set_error(why);
    return rc;
  }
  int64_t total = 0;
  try {
    std::vector<Run> runs;
    build_runs(g, dev_idx, host_idx, n, &runs);
    total = (int64_t)runs.size() * (int64_t)(l1 - l0) * g.C;
    if (merge2d) {
      std::vector<Copy> copies;
      build_copies(g, runs, dev_idx, host_idx, &copies);
      // a 2-D copy whose region would leave the host pool or the device
      // buffer sends its last line as a call of its own (copy_calls)
      total = 0;
      for (const Copy &c : copies) {
        if (c.lines == 1) {
          total += (int64_t)(l1 - l0) * g.C;
          continue;
        }
        for (int64_t lc = (int64_t)l0 * g.C; lc < (int64_t)l1 * g.C; lc++)
          total += copy_calls(g, c, lc);
      }
    }
  } catch (const std::bad_alloc &) {
    set_error("out of host memory while counting segments");
    return KV_ENOMEM;
  }
  *out = total;
  return KV_OK;
}

extern "C" int kv_count_segments(const kv_geometry_t *geom, const int64_t *dev_idx,
                                 const int64_t *host_idx, int64_t n, int32_t layer_begin,
                                 int32_t layer_end, int64_t *out) {
  return count_common(geom, dev_idx, host_idx, n, layer_begin, layer_end, out, false);
}

extern "C" int kv_count_dma_copies(const kv_geometry_t *geom, const int64_t *dev_idx,
                                   const int64_t *host_idx, int64_t n, int32_t layer_begin,
                                   int32_t layer_end, int64_t *out) {
  return count_common(geom, dev_idx, host_idx, n, layer_begin, layer_end, out, true);
}
