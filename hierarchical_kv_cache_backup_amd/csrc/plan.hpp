// plan.hpp — host-side planner of the cross-tier KV transfer (no HIP).
//
// Every host layout's address map splits into a per-(layer, component) part
// and a per-token part:
//   host_row(l, c, h) = (l*C + c) * lc_stride + host_key(h)
//   layer_first        lc_stride = S_host   host_key(h) = h
//   page_first         lc_stride = 1        host_key(h) = h * L*C
//   page_first_direct  lc_stride = ps       host_key(h) = (h / ps) * L*C*ps + h % ps
// (dimension orders from "Tuning SGLang HiCache L2 on Kunlunxin P800/P900",
// section 2.1, and "HiCache system design", section "data transfer
// optimisation"; the component axis sits directly inside the layer axis).
// Because of this split, whether two consecutive request positions are
// contiguous on the host does not depend on (l, c), so the run structure of a
// request is computed once per call, in O(n), and reused for every (l, c).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kvtier.h"

namespace kvt {

// Largest row the library takes: the kernels count a row's chunks in 32 bits
// (8-byte chunks on the direct path), and a staged launch holds at least
// stage_max_rows(R) >= 32 rows.
constexpr int64_t kRowBytesLimit = int64_t(1) << 30;

struct Geom {
  int32_t L = 0, C = 0;
  int64_t R = 0, S_dev = 0, S_host = 0;
  int32_t ps = 1, layout = KV_LAYER_FIRST;
  int64_t lc_stride = 0;  // host rows between (l,c) and the next (l,c)
};

// Checks the geometry and fills g (lc_stride included). On failure returns
// KV_EINVAL and writes a reason to *why.
int make_geom(const kv_geometry_t *in, Geom *g, std::string *why);

inline int64_t host_key(const Geom &g, int64_t h) {
  switch (g.layout) {
    case KV_LAYER_FIRST:
      return h;
    case KV_PAGE_FIRST:
      return h * (int64_t)g.L * g.C;
    default: {
      const int64_t q = h / g.ps;
      return q * (int64_t)g.L * g.C * g.ps + (h - q * g.ps);
    }
  }
}

inline int64_t host_row(const Geom &g, int32_t l, int32_t c, int64_t h) {
  return ((int64_t)l * g.C + c) * g.lc_stride + host_key(g, h);
}

// Reusable scratch for the O(n) destination-uniqueness check: one stamp per
// slot and a generation counter, so no clearing between calls. Used while the
// pool has at most max(kStampSlotsMin, 4 n) destination slots; beyond that the
// check sorts a copy of the request instead (O(n log n), no per-slot memory).
// A table that already covers the pool's slots is always used. A pool made
// with the uniqueness check sizes its tables at creation for up to
// kStampSlotsPresize slots, so that kv_transfer_noalloc can check without
// allocating.
constexpr int64_t kStampSlotsMin = int64_t(1) << 22;
constexpr int64_t kStampSlotsPresize = int64_t(1) << 24;  // 64 MiB per direction at most
struct UniqueScratch {
  std::vector<uint32_t> stamp;
  uint32_t gen = 0;
};

// Request validation (rules and their order are those documented for
// kv_validate). `scratch` may be null when check_unique is false. Without
// may_allocate the uniqueness check uses only a table that already covers the
// destination slots (else KV_EINVAL): on success nothing is allocated.
int validate(const Geom &g, int direction, const int64_t *dev_idx, const int64_t *host_idx,
             int64_t n, int32_t l0, int32_t l1, bool check_unique, UniqueScratch *scratch,
             std::string *why, bool may_allocate = true);

// Validation of kv_stage (the staged path's device-side pass on its own): the
// rules of validate without the host side. Only an unpack (direction 1) writes
// device slots, so only it checks them for repeats.
int validate_stage(const Geom &g, int direction, const int64_t *dev_idx, int64_t n, int32_t l0,
                   int32_t l1, bool check_unique, UniqueScratch *scratch, std::string *why);

// A maximal group of request positions [i0, i0+len) whose device slots and
// host rows both advance by one row per position.
struct Run {
  int64_t i0, len;
};

// Runs of the request, in request order (identical for every (l, c)).
void build_runs(const Geom &g, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                std::vector<Run> *runs);

// One copy-engine call, relative to (l, c): `lines` lines of `len` rows each;
// line j starts at device slot dev0 + j*dev_pitch and host key key0 + j*key_pitch
// (both in rows). lines == 1 means a plain 1-D copy.
struct Copy {
  int64_t dev0, key0, len, lines, dev_pitch, key_pitch;
};

// Merges consecutive runs of equal length at constant device and host pitch
// (pitch >= len, so lines never overlap) into 2-D copies.
void build_copies(const Geom &g, const std::vector<Run> &runs, const int64_t *dev_idx,
                  const int64_t *host_idx, std::vector<Copy> *copies);

// A 2-D copy-engine call names a region of pitch x lines bytes on each side,
// although its last line is only len rows long. Lines of copy c on (layer,
// component) buffer lc that can go out as one 2-D call whose whole region lies
// inside the host pool (L*C*S_host rows) and inside the device buffer (S_dev
// rows): min(lines, lines that fit on each side). Every line itself lies
// inside both, so at most the last line is left over; it goes out as a 1-D
// copy. 1 for a 1-D copy.
inline int64_t copy_region_lines(const Geom &g, const Copy &c, int64_t lc) {
  if (c.lines <= 1) return c.lines;
  const int64_t host_rows = (int64_t)g.L * g.C * g.S_host;
  const int64_t fit_h = (host_rows - (lc * g.lc_stride + c.key0)) / c.key_pitch;
  const int64_t fit_d = (g.S_dev - c.dev0) / c.dev_pitch;
  const int64_t fit = fit_h < fit_d ? fit_h : fit_d;
  return fit < c.lines ? fit : c.lines;
}

// Copy-engine calls copy c takes on buffer lc: one 2-D call over the lines
// copy_region_lines allows (when that is 2 or more) and one 1-D call per line
// left, else one 1-D call per line.
inline int64_t copy_calls(const Geom &g, const Copy &c, int64_t lc) {
  const int64_t fit = copy_region_lines(g, c, lc);
  return fit >= 2 ? 1 + (c.lines - fit) : c.lines;
}

// Staged path: the rows (i, l, c), l in [la, lb), are enumerated in the
// transfer kernels' host-order walk (groups of G request positions, then
// (pair, position) inside a group; G = n, 1 or page_size for layer_first,
// page_first, page_first_direct). A staging buffer holds walk row r at
// r * R. An extent is a maximal range of walk rows whose host rows are
// consecutive: one copy-engine call moves it between the staging buffer and
// the host pool.
struct Extent {
  int64_t walk0, host0, rows;
};

// Extents of the walk over layers [la, lb), in walk order. Cost O(n) plus
// O(pairs x host runs) (one pass per pair over the runs of consecutive host
// slots), and O(n) for page_first whose token rows are contiguous.
void build_extents(const Geom &g, const int64_t *host_idx, int64_t n, int32_t la, int32_t lb,
                   std::vector<Extent> *out);

// The same in two steps, so that a call split into layer groups finds the runs
// of host-consecutive positions once (O(n)) and then pays O(pairs x runs) per
// group: host_runs writes the first position of every run and then n.
void host_runs(const Geom &g, const int64_t *host_idx, int64_t n, std::vector<int64_t> *start);
void build_extents(const Geom &g, const int64_t *host_idx, int64_t n,
                   const std::vector<int64_t> &run_start, int32_t la, int32_t lb,
                   std::vector<Extent> *out);

// Chunk lengths (rows, in walk order) of a staged unit of walk_rows rows
// through staging halves of chunk_rows rows. A chunk fills a half, except
// where its device-side pass has no copy to overlap: a write-back's first
// gather (nothing is ready to copy out yet; ramp_first) and a call's last
// scatter (nothing is left to copy in; ramp_last). There the chunks grow from
// 1/kRampFirst of a half by kRampGrowth per chunk (ascending at the start,
// mirrored at the end), so the pass that runs alone is short. Each ramp
// chunk's copy over the host link outlasts the next chunk's pass in HBM (the
// passes run >10x the link rate), so the ramp adds launches and copies but no
// stall.
constexpr int64_t kRampFirst = 64, kRampGrowth = 8;
void chunk_plan(int64_t walk_rows, int64_t chunk_rows, bool ramp_first, bool ramp_last,
                std::vector<int64_t> *out);

}  // namespace kvt
