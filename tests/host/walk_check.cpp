// walk_check.cpp — CPU replay of the library's launch plans against the oracle.
//
// Built with the host compiler under AddressSanitizer/UBSan by
// tests/test_host_planner.py. For random geometries and requests it replays,
// on host mirrors of the device pool and of the host pool:
//   * every workgroup/lane/unroll step of the direct kernel (xfer_rows), with
//     the same constexpr walk the kernel runs (xfer_walk.hpp), for one launch
//     over all layers and for per-layer launches;
//   * every tile, phase and LDS slot of the LDS-staged kernel;
//   * every copy of the copy-engine plan (runs merged into 2-D copies);
// and checks that each chunk of each row is moved exactly once, that
// every address and LDS slot stays in bounds, and that the resulting bytes equal
// the oracle's. It also checks the segment counter against the oracle's.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "kvtier.h"
#include "plan.hpp"
#include "xfer_walk.hpp"

extern "C" {
int kvo_backup(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
               uint8_t *const *dev_bufs, uint8_t *host, const int64_t *dev_idx,
               const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique);
int kvo_load(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps, int layout,
             uint8_t *const *dev_bufs, const uint8_t *host, const int64_t *dev_idx,
             const int64_t *host_idx, int64_t n, int l0, int l1, int check_unique);
int64_t kvo_count_segments(int L, int C, int64_t R, int64_t S_dev, int64_t S_host, int ps,
                           int layout, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                           int l0, int l1);
}

namespace kvt {
void set_error(const std::string &) {}
}

using namespace kvt;

static int failures = 0;
static int64_t regions_split = 0;  // 2-D copies whose last line went out on its own
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (failures < 20) {                                 \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);                 \
        std::fprintf(stderr, "\n");                        \
      }                                                    \
      failures++;                                          \
    }                                                      \
  } while (0)

struct Mirror {
  Geom g;
  std::vector<std::vector<uint8_t>> dev;  // L*C buffers
  std::vector<uint8_t> host;
  std::vector<uint8_t *> ptrs() {
    std::vector<uint8_t *> p;
    for (auto &b : dev) p.push_back(b.data());
    return p;
  }
};

// Replays one launch of xfer_rows on the mirrors, `depth` chunks in flight per
// lane. tok holds {dev slot, host key}. Like the kernel, a slot past the
// block's chunks resolves the block's last chunk (its index loads must stay in
// bounds) and moves nothing (the kernel sends it to its sink).
static void replay_rows(Mirror &m, const std::vector<int64_t> &tok, int64_t n, int32_t la,
                        int32_t lb, bool to_host, std::vector<uint8_t> &cover, uint32_t cap,
                        int depth) {
  const Geom &g = m.g;
  XferArgs a{};
  a.R = g.R;
  a.lc_stride = g.lc_stride;
  a.n = (uint32_t)n;
  a.lc0 = (uint32_t)(la * g.C);
  a.nlc = (uint32_t)((lb - la) * g.C);
  const uint32_t blocks = plan_rows(&a, g.layout, g.ps);
  CHECK((uint64_t)blocks * a.rows_per_block >= a.total_rows, "grid too small");
  CHECK(blocks == 0 || (uint64_t)(blocks - 1) * a.rows_per_block < a.total_rows, "idle block");
  CHECK(a.nblocks == blocks, "nblocks");
  const uint32_t grid = grid_for(blocks, cap);
  CHECK(grid >= 1 && grid <= blocks, "grid %u for %u blocks", grid, blocks);
  for (uint32_t wg = 0; wg < grid; wg++)
  for (uint32_t b = wg; b < a.nblocks; b += grid) {
    const uint32_t row0 = b * a.rows_per_block;
    const uint32_t nrows = umin(a.rows_per_block, a.total_rows - row0);
    const uint32_t nchunks = nrows * a.cpr;
    for (uint32_t base = 0; base < nchunks; base += (uint32_t)kXferThreads * depth)
      for (int u = 0; u < depth; u++)
        for (uint32_t tid = 0; tid < (uint32_t)kXferThreads; tid++) {
          const uint32_t f0 = base + u * kXferThreads + tid;
          const bool live = f0 < nchunks;
          const uint32_t f = live ? f0 : nchunks - 1;
          const uint32_t rr = f / a.cpr, k = f - rr * a.cpr;
          uint32_t i = 0, lc = 0;
          walk_row(a, row0 + rr, i, lc);
          CHECK(i < a.n && lc < a.nlc, "walk out of range i=%u lc=%u", i, lc);
          if (!(i < a.n && lc < a.nlc)) return;
          const int64_t dslot = tok[2 * i], key = tok[2 * i + 1];
          const int64_t dev_off = dslot * g.R + kChunkBytes * (int64_t)k;
          const int64_t host_off = ((int64_t)(a.lc0 + lc) * a.lc_stride + key) * g.R + kChunkBytes * (int64_t)k;
          CHECK(dev_off >= 0 && dev_off + kChunkBytes <= g.S_dev * g.R, "device offset out of bounds");
          CHECK(host_off >= 0 && host_off + kChunkBytes <= (int64_t)m.host.size(), "host offset out of bounds");
          if (!live) continue;
          uint8_t *d = m.dev[a.lc0 + lc].data() + dev_off;
          uint8_t *h = m.host.data() + host_off;
          if (to_host)
            std::memcpy(h, d, kChunkBytes);
          else
            std::memcpy(d, h, kChunkBytes);
          const int64_t cell = ((int64_t)i * g.L * g.C + a.lc0 + lc) * a.cpr + k;
          cover[cell]++;
        }
  }
}

// Replays one launch of xfer_tiles_lds.
static void replay_tiles(Mirror &m, const std::vector<int64_t> &tok, int64_t n, int32_t la,
                         int32_t lb, bool to_host, std::vector<uint8_t> &cover, uint32_t cap) {
  const Geom &g = m.g;
  XferArgs a{};
  a.R = g.R;
  a.lc_stride = g.lc_stride;
  a.n = (uint32_t)n;
  a.lc0 = (uint32_t)(la * g.C);
  a.nlc = (uint32_t)((lb - la) * g.C);
  plan_rows(&a, g.layout, g.ps);
  TileArgs ta{};
  a.nblocks = plan_tiles(a, g.layout, &ta);
  const size_t lds_bytes = (size_t)ta.tile_t * ta.tile_lc * g.R;
  CHECK(lds_bytes <= 64 * 1024, "LDS tile of %zu bytes exceeds 64 KiB", lds_bytes);
  std::vector<uint8_t> lds(lds_bytes);
  const uint32_t grid = grid_for(a.nblocks, cap);
  for (uint32_t wg = 0; wg < grid; wg++)
  for (uint32_t b = wg; b < a.nblocks; b += grid) {
    const Tile t = tile_of(a, ta, b);
    CHECK(t.nt >= 1 && t.nl >= 1 && t.i0 + t.nt <= a.n && t.lcf + t.nl <= a.nlc, "bad tile");
    const uint32_t nchunks = t.nt * t.nl * a.cpr;
    const bool host_pm = ta.token_major != 0;
    for (int phase = 0; phase < 2; phase++) {
      const bool pos_major = phase == 0 ? (to_host ? false : host_pm) : (to_host ? host_pm : false);
      for (uint32_t f = 0; f < nchunks; f++) {
        uint32_t lc_t = 0, p_t = 0, k = 0;
        tile_walk(t, a.cpr, pos_major, f, lc_t, p_t, k);
        const uint32_t slot = tile_slot(t, a.cpr, lc_t, p_t, k);
        CHECK((size_t)slot * kChunkBytes + kChunkBytes <= lds_bytes, "LDS slot out of bounds");
        const uint32_t i = t.i0 + p_t, lc = t.lcf + lc_t;
        const int64_t dev_off = tok[2 * i] * g.R + kChunkBytes * (int64_t)k;
        const int64_t host_off =
            ((int64_t)(a.lc0 + lc) * a.lc_stride + tok[2 * i + 1]) * g.R + kChunkBytes * (int64_t)k;
        CHECK(host_off >= 0 && host_off + kChunkBytes <= (int64_t)m.host.size(), "host offset OOB");
        uint8_t *d = m.dev[a.lc0 + lc].data() + dev_off;
        uint8_t *h = m.host.data() + host_off;
        uint8_t *s = lds.data() + (size_t)slot * kChunkBytes;
        if (phase == 0) {
          std::memcpy(s, to_host ? d : h, kChunkBytes);
        } else {
          std::memcpy(to_host ? h : d, s, kChunkBytes);
          cover[((int64_t)i * g.L * g.C + a.lc0 + lc) * a.cpr + k]++;
        }
      }
    }
  }
}

// Replays the staged path over layers [la, lb): extents of the walk, then the
// chunks of chunk_plan (halves of chunk_rows rows, ramped as asked) with the
// dense gather (D2H) or scatter (H2D) through a staging mirror and one memcpy
// per extent piece, as the executor issues them.
static void replay_staged(Mirror &m, const std::vector<int64_t> &tok, const int64_t *h, int64_t n,
                          int32_t la, int32_t lb, bool to_host, std::vector<uint8_t> &cover,
                          int64_t chunk_rows, bool ramp_first, bool ramp_last,
                          uint32_t cap, uint32_t step) {
  const Geom &g = m.g;
  XferArgs a{};
  a.R = g.R;
  a.lc_stride = g.lc_stride;
  a.n = (uint32_t)n;
  a.lc0 = (uint32_t)(la * g.C);
  a.nlc = (uint32_t)((lb - la) * g.C);
  plan_rows(&a, g.layout, g.ps);
  std::vector<Extent> ext;
  build_extents(g, h, n, la, lb, &ext);
  // extents tile the walk in order, and map every walk row to its host row
  int64_t next = 0;
  for (const Extent &e : ext) {
    CHECK(e.walk0 == next && e.rows > 0, "extent gap or overlap at walk row %lld", (long long)next);
    for (int64_t r = e.walk0; r < e.walk0 + e.rows; r++) {
      uint32_t i = 0, lc = 0;
      walk_row(a, (uint32_t)r, i, lc);
      const int64_t want = (int64_t)(a.lc0 + lc) * g.lc_stride + tok[2 * i + 1];
      CHECK(e.host0 + (r - e.walk0) == want, "extent maps walk row %lld wrong", (long long)r);
    }
    next = e.walk0 + e.rows;
  }
  CHECK(next == (int64_t)a.total_rows, "extents cover %lld of %u rows", (long long)next,
        a.total_rows);
  std::vector<int64_t> chunks;
  chunk_plan(a.total_rows, chunk_rows, ramp_first, ramp_last, &chunks);
  int64_t sum = 0;
  for (size_t k = 0; k < chunks.size(); k++) {
    CHECK(chunks[k] >= 1 && chunks[k] <= chunk_rows, "chunk of %lld rows (half %lld)",
          (long long)chunks[k], (long long)chunk_rows);
    // a ramp grows by kRampGrowth at most per chunk, towards the full half
    if (ramp_first && k + 1 < chunks.size())
      CHECK(chunks[k + 1] <= chunks[k] * kRampGrowth, "ramp grows too fast");
    sum += chunks[k];
  }
  CHECK(sum == (int64_t)a.total_rows, "chunks cover %lld of %u rows", (long long)sum,
        a.total_rows);
  if (ramp_first || ramp_last) {
    const int64_t edge = ramp_first ? chunks.front() : chunks.back();
    CHECK(edge <= std::max<int64_t>(1, chunk_rows / kRampFirst), "ramp starts at %lld rows",
          (long long)edge);
  }
  std::vector<uint8_t> stage((size_t)(chunk_rows * g.R));
  size_t x = 0;
  int64_t r0 = 0;
  for (int64_t len : chunks) {
    const int64_t r1 = r0 + len;
    set_row_range(&a, (uint32_t)r0, (uint32_t)r1);
    // the device-side pass (stage_windows): wave w of the grid-stride loop
    // moves window w of the staging chunk stream; lane `lane` moves chunk k of
    // the window's row j (stage_lane). Wide rows: the wave resolves the
    // window's first row with walk_at and the second with walk_next. Narrow
    // rows: lane j resolves row ra + j with walk_at, for j < rows.
    auto window_pass = [&](const XferArgs &piece, bool gather) {
      const uint32_t cpr16 = stage_cpr(g.R);
      const bool wide = stage_wide(g.R);
      const uint32_t recip = stage_recip_of(g.R);
      CHECK(stage_chunks(piece) == (uint64_t)(piece.row_end - piece.row_begin) * cpr16 &&
                (uint64_t)(piece.row_end - piece.row_begin) * cpr16 <= kStageMaxChunks,
            "stage chunk count");
      const uint32_t nwin = stage_windows(piece);
      const uint32_t grid = grid_for(stage_blocks(piece), cap);
      CHECK((uint64_t)stage_blocks(piece) * kWavesPerBlock >= nwin, "stage grid too small");
      const uint32_t total = stage_chunks(piece);
      for (uint32_t b = 0; b < grid; b++)
        for (uint32_t wave = 0; wave < kWavesPerBlock; wave++)
          for (uint32_t w = b * kWavesPerBlock + wave; w < nwin; w += grid * kWavesPerBlock) {
            const StageWindow s = stage_window(piece, w, recip);
            CHECK(s.rows >= 1 && s.rows <= (wide ? 2u : 64u), "window of %u rows", s.rows);
            if (s.rows < 1 || s.rows > 64) return;
            // the rows' (position, pair) as the kernel resolves them
            uint32_t ri[64], rl[64];
            if (wide) {
              WalkPos wp = walk_at(piece, piece.row_begin + s.ra);
              ri[0] = wp.base + wp.pos;
              rl[0] = wp.lc;
              if (s.rows > 1) {
                walk_next(piece, wp);
                ri[1] = wp.base + wp.pos;
                rl[1] = wp.lc;
              }
            } else {
              for (uint32_t jj = 0; jj < s.rows; jj++) {
                const WalkPos wp = walk_at(piece, piece.row_begin + s.ra + jj);
                ri[jj] = wp.base + wp.pos;
                rl[jj] = wp.lc;
              }
            }
            for (uint32_t jj = 0; jj < s.rows; jj++) {
              uint32_t i = 0, lc = 0;
              walk_row(piece, piece.row_begin + s.ra + jj, i, lc);
              CHECK(ri[jj] == i && rl[jj] == lc, "window row %u of window %u differs", jj, w);
              CHECK(i < piece.n && lc < piece.nlc, "stage walk out of range");
              if (!(i < piece.n && lc < piece.nlc)) return;
            }
            for (uint32_t lane = 0; lane < 64; lane++) {
              const uint32_t c = s.c0 + lane;
              if (c >= total) continue;
              uint32_t jj = 0, k = 0;
              stage_lane(s, cpr16, recip, lane, jj, k);
              if (wide) {  // the kernel's form of the same mapping
                const uint32_t split = cpr16 - s.ka;
                CHECK(lane < split ? (jj == 0 && k == s.ka + lane) : (jj == 1 && k == lane - split),
                      "wide lane %u of window %u: compare form differs", lane, w);
              }
              CHECK(jj < s.rows && k < cpr16 && (s.ra + jj) * cpr16 + k == c,
                    "lane %u of window %u maps to row %u chunk %u", lane, w, jj, k);
              if (!(jj < s.rows && k < cpr16)) return;
              const uint32_t i = ri[jj], lc = rl[jj];
              const bool inside = piece.host >= stage.data() &&
                                  piece.host - stage.data() + (int64_t)(c + 1) * 16 <=
                                      (int64_t)stage.size();
              CHECK(inside, "stage overrun");
              if (!inside) return;
              uint8_t *dv = m.dev[piece.lc0 + lc].data() + tok[2 * i] * g.R + 16 * (int64_t)k;
              uint8_t *sv = piece.host + 16 * (int64_t)c;
              if (gather)
                std::memcpy(sv, dv, 16);
              else
                std::memcpy(dv, sv, 16);
              for (int h8 = 0; h8 < 2; h8++)
                cover[((int64_t)i * g.L * g.C + piece.lc0 + lc) * (g.R / kChunkBytes) + 2 * k + h8]++;
            }
          }
    };
    // launch_stage splits the pass into pieces of at most `step` rows
    // (stage_piece; stage_max_rows(R) in the library, small steps here too)
    auto dense = [&](bool gather) {
      XferArgs whole = a;
      whole.host = stage.data();
      for (uint32_t r = whole.row_begin; r < whole.row_end; r += step) {
        const XferArgs p = stage_piece(whole, r, step);
        const bool ok = p.row_begin == r && p.row_end > r && p.row_end <= whole.row_end &&
                        p.host == stage.data() + (int64_t)(r - whole.row_begin) * g.R;
        CHECK(ok, "stage piece at row %u", r);
        if (ok) window_pass(p, gather);
      }
    };
    if (to_host) dense(true);
    while (x < ext.size() && ext[x].walk0 < r1) {
      const Extent &e = ext[x];
      const int64_t a0 = std::max(e.walk0, r0), a1 = std::min(e.walk0 + e.rows, r1);
      const int64_t host_off = (e.host0 + (a0 - e.walk0)) * g.R;
      CHECK(host_off >= 0 && host_off + (a1 - a0) * g.R <= (int64_t)m.host.size(), "extent OOB");
      uint8_t *hp = m.host.data() + host_off;
      uint8_t *sp = stage.data() + (a0 - r0) * g.R;
      if (to_host)
        std::memcpy(hp, sp, (a1 - a0) * g.R);
      else
        std::memcpy(sp, hp, (a1 - a0) * g.R);
      if (e.walk0 + e.rows > r1) break;
      x++;
    }
    if (!to_host) dense(false);
    r0 = r1;
  }
}

// Executes the copy-engine plan with memcpy, line by line.
static void replay_dma(Mirror &m, const int64_t *d, const int64_t *h, int64_t n, int32_t l0,
                       int32_t l1, bool to_host, int64_t *copies_out) {
  const Geom &g = m.g;
  std::vector<Run> runs;
  std::vector<Copy> copies;
  build_runs(g, d, h, n, &runs);
  build_copies(g, runs, d, h, &copies);
  int64_t total = 0;
  for (const Run &r : runs) total += r.len;
  CHECK(total == n, "runs cover %lld of %lld positions", (long long)total, (long long)n);
  int64_t calls = 0;
  for (int32_t l = l0; l < l1; l++)
    for (int32_t c = 0; c < g.C; c++)
      for (const Copy &cp : copies) {
        CHECK(cp.lines == 1 || (cp.dev_pitch >= cp.len && cp.key_pitch >= cp.len), "bad pitch");
        // the region a 2-D call names is pitch x height on each side: it must lie
        // inside the host pool and the device buffer, not only its lines
        const int64_t lc = (int64_t)l * g.C + c;
        const int64_t region = copy_region_lines(g, cp, lc);
        CHECK(region >= 1 && region <= cp.lines && region >= cp.lines - 1,
              "2-D region of %lld lines for a copy of %lld", (long long)region,
              (long long)cp.lines);
        if (region >= 2) {
          const int64_t host_end = (lc * g.lc_stride + cp.key0 + region * cp.key_pitch) * g.R;
          const int64_t dev_end = (cp.dev0 + region * cp.dev_pitch) * g.R;
          CHECK(host_end <= (int64_t)m.host.size(), "2-D host region ends %lld bytes past the pool",
                (long long)(host_end - (int64_t)m.host.size()));
          CHECK(dev_end <= g.S_dev * g.R, "2-D device region ends %lld bytes past the buffer",
                (long long)(dev_end - g.S_dev * g.R));
          if (region < cp.lines) regions_split++;
        }
        calls += copy_calls(g, cp, lc);
        for (int64_t j = 0; j < cp.lines; j++) {
          const int64_t dev_off = (cp.dev0 + j * cp.dev_pitch) * g.R;
          const int64_t host_off = ((int64_t)(l * g.C + c) * g.lc_stride + cp.key0 + j * cp.key_pitch) * g.R;
          const int64_t w = cp.len * g.R;
          CHECK(dev_off >= 0 && dev_off + w <= g.S_dev * g.R, "DMA device range OOB");
          CHECK(host_off >= 0 && host_off + w <= (int64_t)m.host.size(), "DMA host range OOB");
          uint8_t *dp = m.dev[l * g.C + c].data() + dev_off;
          uint8_t *hp = m.host.data() + host_off;
          if (to_host)
            std::memcpy(hp, dp, w);
          else
            std::memcpy(dp, hp, w);
        }
      }
  *copies_out = calls;
}

// Replays every executor's plan of one request (both directions) on CPU
// mirrors and compares the bytes with the oracle's.
static int64_t check_case(const kv_geometry_t &kg, const Geom &g, const std::vector<int64_t> &d,
                          const std::vector<int64_t> &h, int32_t l0, int32_t l1, int cs,
                          std::mt19937_64 &rng) {
  auto uni = [&](int64_t lo, int64_t hi) {  // inclusive
    return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
  };
  const int64_t n = (int64_t)d.size();
  const int64_t nlc = (int64_t)(l1 - l0) * g.C;
  int64_t checked = 0;
  Mirror base;
  base.g = g;
  base.dev.resize((size_t)g.L * g.C);
  for (auto &b : base.dev) {
    b.resize((size_t)(g.S_dev * g.R));
    for (auto &x : b) x = (uint8_t)rng();
  }
  base.host.resize((size_t)((int64_t)g.L * g.C * g.S_host * g.R));
  for (auto &x : base.host) x = (uint8_t)rng();

  // expected results from the oracle
  Mirror want_b = base, want_l = base;
  {
    auto p = want_b.ptrs();
    CHECK(kvo_backup(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout, p.data(),
                     want_b.host.data(), d.data(), h.data(), n, l0, l1, 1) == 0, "oracle backup");
    auto q = want_l.ptrs();
    CHECK(kvo_load(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout, q.data(),
                   want_l.host.data(), d.data(), h.data(), n, l0, l1, 1) == 0, "oracle load");
  }
  int64_t seg = -1;
  CHECK(kv_count_segments(&kg, d.data(), h.data(), n, l0, l1, &seg) == KV_OK, "count");
  CHECK(seg == kvo_count_segments(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout, d.data(),
                                  h.data(), n, l0, l1),
        "segment count differs from the oracle");

  std::vector<int64_t> tok(2 * (size_t)n);
  for (int64_t i = 0; i < n; i++) {
    tok[2 * i] = d[i];
    tok[2 * i + 1] = host_key(g, h[i]);
  }
  const int64_t cells = n * g.L * g.C * (g.R / kChunkBytes);
  for (int dir = 0; dir < 2; dir++) {
    const bool to_host = dir == 0;
    const Mirror &want = to_host ? want_b : want_l;
    for (int variant = 0; variant < 5; variant++) {
      if (n == 0 || nlc == 0) break;
      if (variant == 2 && g.R > kMaxLdsRowBytes) continue;
      Mirror m = base;
      std::vector<uint8_t> cover((size_t)cells, 0);
      int64_t copies = 0;
      const uint32_t cap = (uint32_t)(std::vector<int>{0, 1, 3, 64})[uni(0, 3)];
      const int depth = (std::vector<int>{1, 2, 4, 8})[uni(0, 3)];
      if (variant == 0) {
        replay_rows(m, tok, n, l0, l1, to_host, cover, cap, depth);
      } else if (variant == 1) {
        for (int32_t l = l0; l < l1; l++)
          replay_rows(m, tok, n, l, l + 1, to_host, cover, cap, depth);
      } else if (variant == 2) {
        replay_tiles(m, tok, n, l0, l1, to_host, cover, cap);
      } else if (variant == 4) {
        const int64_t walk = n * (int64_t)(l1 - l0) * g.C;
        const int64_t chunk = std::max<int64_t>(1, (std::vector<int64_t>{1, 7, walk / 3 + 1, walk})[uni(0, 3)]);
        const int ramp = (int)uni(0, 2);  // none, first, last
        // pieces of the library's size, or small ones that split every chunk
        const uint32_t step = uni(0, 1) ? stage_max_rows(g.R) : (uint32_t)uni(1, 40);
        replay_staged(m, tok, h.data(), n, l0, l1, to_host, cover, chunk, ramp == 1, ramp == 2,
                      cap, step);
      } else {
        replay_dma(m, d.data(), h.data(), n, l0, l1, to_host, &copies);
        int64_t counted = -1;
        CHECK(kv_count_dma_copies(&kg, d.data(), h.data(), n, l0, l1, &counted) == KV_OK &&
                  counted == copies,
              "dma copy count");
        CHECK(copies <= seg, "more copies than segments");
      }
      if (variant != 3) {  // every kernel-driven variant moves each chunk exactly once
        for (int64_t i = 0; i < n; i++)
          for (int32_t lc = 0; lc < g.L * g.C; lc++)
            for (int64_t k = 0; k < g.R / kChunkBytes; k++) {
              const bool inside = lc >= l0 * g.C && lc < l1 * g.C;
              const uint8_t cnt = cover[(size_t)((i * g.L * g.C + lc) * (g.R / kChunkBytes) + k)];
              CHECK(cnt == (inside ? 1 : 0), "chunk moved %d times (variant %d)", cnt, variant);
            }
      }
      CHECK(m.host == want.host, "host pool differs from oracle (case %d dir %d variant %d)", cs,
            dir, variant);
      for (size_t b = 0; b < m.dev.size(); b++)
        CHECK(m.dev[b] == want.dev[b], "device buffer %zu differs (case %d dir %d variant %d)", b,
              cs, dir, variant);
      checked++;
    }
  }
  return checked;
}

int main(int argc, char **argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) {  // inclusive
    return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
  };
  int64_t checked = 0;
  // Directed: uniform-pitch runs that end at the last host slot or device slot,
  // so a 2-D copy's pitch x height region would run past the host pool or the
  // device buffer although its last line fits: runs of 16 slots at pitch 32
  // from slot 16 (layer_first, the region ends past both), and a request on the
  // last 4 pages of a page_first_direct pool of 78 layers (past the host pool).
  {
    struct Directed {
      int32_t L, C, ps, layout;
      int64_t R, S_dev, S_host;
    };
    const Directed cases_d[] = {{3, 2, 16, 0, 48, 640, 640}, {78, 1, 64, 2, 16, 256, 512}};
    for (int k = 0; k < 2; k++) {
      const Directed &x = cases_d[k];
      const kv_geometry_t kg{x.L, x.C, x.R, x.S_dev, x.S_host, x.ps, x.layout};
      Geom g;
      std::string why;
      CHECK(make_geom(&kg, &g, &why) == KV_OK, "directed geometry: %s", why.c_str());
      std::vector<int64_t> d, h;
      if (k == 0) {
        for (int64_t s0 = 16; s0 + 16 <= 640; s0 += 32)
          for (int64_t j = 0; j < 16; j++) d.push_back(s0 + j);
        h = d;
      } else {
        for (int64_t j = 0; j < 256; j++) {
          d.push_back(j);
          h.push_back(256 + j);
        }
      }
      const int64_t before = regions_split;
      checked += check_case(kg, g, d, h, 0, x.L, -1 - k, rng);
      CHECK(regions_split > before, "directed case %d split no 2-D region", k);
    }
  }
  for (int cs = 0; cs < cases; cs++) {
    kv_geometry_t kg{};
    kg.num_layers = (int32_t)uni(1, 5);
    kg.num_components = (int32_t)uni(1, 2);
    // row sizes on both sides of the staged pass's window (64 chunks, 1 KiB):
    // narrow rows that do and do not divide it, the widest narrow row (1008),
    // a row of exactly one window (1024), wide rows that straddle windows;
    // the first cases take each size once, the others draw
    const int64_t sizes[] = {16, 48, 256, 272, 512, 528, 1008, 1024, 1040, 1152, 2048, 36864};
    const int nsizes = (int)(sizeof(sizes) / sizeof(sizes[0]));
    kg.row_bytes = cs < nsizes ? sizes[cs] : sizes[uni(0, nsizes - 1)];
    kg.page_size = (int32_t)(std::vector<int>{1, 2, 3, 4, 16, 64})[uni(0, 5)];
    kg.host_slots = kg.page_size * uni(1, 300 / kg.page_size + 1);
    kg.device_slots = uni(1, 400);
    kg.host_layout = (int32_t)uni(0, 2);
    if (kg.row_bytes > 4096) {  // keep big-row cases small
      kg.host_slots = kg.page_size * uni(1, 3);
      kg.device_slots = uni(1, 8);
    }
    Geom g;
    std::string why;
    if (make_geom(&kg, &g, &why) != KV_OK) {
      CHECK(false, "geometry rejected: %s", why.c_str());
      continue;
    }
    const int64_t nmax = std::min(g.S_dev, g.S_host);
    const int64_t n = uni(0, nmax);
    // destinations unique for both directions: sample without replacement
    std::vector<int64_t> dv(g.S_dev), hv(g.S_host);
    for (int64_t i = 0; i < g.S_dev; i++) dv[i] = i;
    for (int64_t i = 0; i < g.S_host; i++) hv[i] = i;
    const int mode = (int)uni(0, 2);  // 0 random, 1 contiguous, 2 page-shuffled
    if (mode == 0) {
      std::shuffle(dv.begin(), dv.end(), rng);
      std::shuffle(hv.begin(), hv.end(), rng);
    } else if (mode == 1) {
      std::rotate(dv.begin(), dv.begin() + uni(0, g.S_dev - n), dv.end());
    } else {
      std::shuffle(dv.begin(), dv.end(), rng);
      std::sort(dv.begin(), dv.begin() + n);
    }
    std::vector<int64_t> d(dv.begin(), dv.begin() + n), h(hv.begin(), hv.begin() + n);
    const int32_t l0 = (int32_t)uni(0, g.L), l1 = (int32_t)uni(l0, g.L);
    checked += check_case(kg, g, d, h, l0, l1, cs, rng);
  }
  std::printf("walk_check: %lld replays, %lld 2-D regions split, %d failures\n",
              (long long)checked, (long long)regions_split, failures);
  return failures == 0 ? 0 : 1;
}
