// xfer_walk.hpp — launch geometry and index walk of the transfer kernels.
//
// Plain C++ (no HIP types): the functions are constexpr, which clang's HIP
// mode also compiles for the device, so the kernels and the host-side
// checkers run the very same integer arithmetic.
#pragma once

#include <cstdint>

namespace kvt {

// One launch moves the rows (i, lc) for request positions i in [0, n) and
// (layer, component) pairs lc0 + lc, lc in [0, nlc). Rows are enumerated in
// host-address order: groups of G consecutive request positions, and inside a
// group (lc, position) with the position fastest. G = n for layer_first,
// 1 for page_first and page_size for page_first_direct, so consecutive rows of
// the walk are consecutive host rows when the host slots are consecutive.
struct XferArgs {
  const int64_t *tok;       // device: 2 int64 per position, {device slot, host key}
  uint8_t *const *dev_tab;  // device: L*C device buffer base pointers
  uint8_t *host;            // device-visible base address of the host pool
  int64_t R;                // row bytes (multiple of 16)
  int64_t lc_stride;        // host rows between consecutive (layer, component) pairs
  uint32_t n;               // request positions
  uint32_t G;               // group size of the host-order walk
  uint32_t nlc;             // (layer, component) pairs in this launch
  uint32_t lc0;             // first pair = layer_begin * C
  uint32_t cpr;             // chunks (kChunkBytes each) per row
  uint32_t rows_per_block;  // rows one workgroup moves
  uint32_t rows_full;       // rows in complete groups (n / G * G * nlc)
  uint32_t total_rows;      // n * nlc  (< 2^31): rows of the whole walk
  uint32_t row_begin;       // this launch moves walk rows [row_begin, row_end)
  uint32_t row_end;
  uint32_t nblocks;         // row blocks (or LDS tiles); workgroups stride over them
  uint32_t pace_ticks;      // direct kernel: device wall-clock ticks each workgroup takes at
                            // least per block (0 = unpaced)
  uint32_t pace_burst;      // paced: blocks each workgroup moves unpaced before the pacing starts
};

// Tiling of the LDS-staged variant: a workgroup owns tile_t request positions x
// tile_lc pairs (tile_t * tile_lc * R bytes of LDS).
struct TileArgs {
  uint32_t tile_t, tile_lc;
  uint32_t tiles_t, tiles_lc;  // tile counts along positions and pairs
  uint32_t token_major;        // host order is (position, pair): page_first
};

// Each lane moves 8-byte chunks: on gfx950 with mapped host memory, 8-byte
// lanes (non-temporal loads, ordinary stores) keep the host link fuller than
// 16-byte lanes in both directions (measured on contiguous 1 GiB copies).
constexpr int kChunkBytes = 8;
constexpr int kXferThreads = 256;
constexpr int kXferUnroll = 8;                                    // chunks in flight per lane
constexpr uint32_t kChunksPerBlock = kXferThreads * kXferUnroll;  // 16 KiB per workgroup
constexpr uint32_t kLdsTileBytes = 32 * 1024;
constexpr int64_t kMaxLdsRowBytes = 64 * 1024;
constexpr int kLayoutLayerFirst = 0, kLayoutPageFirst = 1, kLayoutPageFirstDirect = 2;

constexpr uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
constexpr uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Fills the derived fields (G, cpr, rows_per_block, rows_full, total_rows)
// from layout, n, nlc and R; returns the number of workgroups.
constexpr uint32_t plan_rows(XferArgs *a, int32_t layout, int32_t page_size) {
  a->G = layout == kLayoutLayerFirst ? a->n
         : layout == kLayoutPageFirst ? 1u
                                      : (uint32_t)page_size;
  a->cpr = (uint32_t)(a->R / kChunkBytes);
  a->rows_per_block = a->cpr >= kChunksPerBlock ? 1u : kChunksPerBlock / a->cpr;
  a->total_rows = a->n * a->nlc;
  a->rows_full = (a->n / a->G) * a->G * a->nlc;
  a->row_begin = 0;
  a->row_end = a->total_rows;
  a->nblocks = (a->total_rows + a->rows_per_block - 1) / a->rows_per_block;
  return a->nblocks;
}

// Restricts a planned launch to walk rows [begin, end); returns the blocks.
constexpr uint32_t set_row_range(XferArgs *a, uint32_t begin, uint32_t end) {
  a->row_begin = begin;
  a->row_end = end;
  a->nblocks = (end - begin + a->rows_per_block - 1) / a->rows_per_block;
  return a->nblocks;
}

// Workgroups to launch for `blocks` blocks of work under a cap (0 = no cap):
// the kernels stride over the blocks, so a capped grid leaves CUs free for
// work on other streams while the host link stays full.
constexpr uint32_t grid_for(uint32_t blocks, uint32_t cap) {
  return (cap == 0 || blocks < cap) ? blocks : cap;
}

// Tile shape of the LDS variant (needs R <= kMaxLdsRowBytes); returns the
// number of workgroups.
constexpr uint32_t plan_tiles(const XferArgs &a, int32_t layout, TileArgs *t) {
  const uint32_t rows_budget = a.R >= kLdsTileBytes ? 1u : (uint32_t)(kLdsTileBytes / a.R);
  t->token_major = layout == kLayoutPageFirst ? 1u : 0u;
  if (t->token_major) {
    t->tile_lc = umin(a.nlc, umax(1u, rows_budget / 4));
    t->tile_t = umin(a.n, umax(1u, rows_budget / t->tile_lc));
  } else {
    t->tile_lc = 1;
    t->tile_t = umin(a.n, rows_budget);
  }
  t->tiles_t = (a.n + t->tile_t - 1) / t->tile_t;
  t->tiles_lc = (a.nlc + t->tile_lc - 1) / t->tile_lc;
  return t->tiles_t * t->tiles_lc;
}

// Request position i and pair lc of row r of the host-order walk.
constexpr void walk_row(const XferArgs &a, uint32_t r, uint32_t &i, uint32_t &lc) {
  if (r < a.rows_full) {
    const uint32_t gsz = a.G * a.nlc;
    const uint32_t grp = r / gsz;
    const uint32_t rem = r - grp * gsz;
    lc = rem / a.G;
    i = grp * a.G + (rem - lc * a.G);
  } else {  // ragged last group (page_first_direct with n % page_size != 0)
    const uint32_t first = a.rows_full / a.nlc;
    const uint32_t t = a.n - first;
    const uint32_t rem = r - a.rows_full;
    lc = rem / t;
    i = first + (rem - lc * t);
  }
}

// Position of a walk row, kept so that the next row's position follows
// without a division (the staged path's device-side pass walks its rows in
// order): request position base + pos, pair lc; gsize positions in the row's
// group (G, or the ragged last group's).
struct WalkPos {
  uint32_t r, base, gsize, pos, lc;
};

constexpr WalkPos walk_at(const XferArgs &a, uint32_t r) {
  WalkPos w{r, 0, 0, 0, 0};
  if (r < a.rows_full) {
    const uint32_t gsz = a.G * a.nlc;
    const uint32_t grp = r / gsz;
    const uint32_t rem = r - grp * gsz;
    w.lc = rem / a.G;
    w.pos = rem - w.lc * a.G;
    w.base = grp * a.G;
    w.gsize = a.G;
  } else {  // needs r < total_rows: the ragged group holds n - first >= 1 positions
    w.base = a.rows_full / a.nlc;
    w.gsize = a.n - w.base;
    const uint32_t rem = r - a.rows_full;
    w.lc = rem / w.gsize;
    w.pos = rem - w.lc * w.gsize;
  }
  return w;
}

// Advances w to the next walk row (the same position walk_row gives it).
constexpr void walk_next(const XferArgs &a, WalkPos &w) {
  w.r++;
  if (w.r == a.rows_full && w.r < a.total_rows) {  // into the ragged last group
    w = walk_at(a, w.r);
    return;
  }
  if (++w.pos == w.gsize) {
    w.pos = 0;
    if (++w.lc == a.nlc) {
      w.lc = 0;
      w.base += w.gsize;
    }
  }
}

// The staged path's device-side pass (stage_windows), HBM to HBM. The staging
// buffer holds the walk rows [row_begin, row_end) back to back, so it is one
// stream of 16-byte chunks: chunk c is chunk c % cpr of walk row
// row_begin + c / cpr (cpr = R / 16). A wave moves one window of kStageWindow
// consecutive chunks (1 KiB: one pass of its 64 lanes), each chunk to or from
// its offset in its device row. Windows are cut on the staging side, not at
// row boundaries, so every pass is full and every wave's staging bytes are one
// aligned KiB whatever the row size. Wide rows (at least kStageWindow chunks):
// a window spans at most two rows, whose device addresses the wave takes once,
// in scalar registers (also rows of exactly half a window, which it holds
// two of). Narrow rows: a window spans up to kStageWindow rows;
// lane j resolves the window's row j, and each lane reads its row's address
// from that lane.
constexpr uint32_t kStageWindow = 64;                     // chunks per window
constexpr uint32_t kWavesPerBlock = kXferThreads / 64;
constexpr uint32_t kStageMaxChunks = uint32_t(1) << 31;   // per launch: chunk numbers fit 32 bits

constexpr uint32_t stage_cpr(int64_t R) { return (uint32_t)(R / 16); }
// Rows whose windows span at most two rows, which the wave resolves in scalar
// registers: rows of a window or more, and rows of exactly half a window (a
// window then holds two whole rows).
constexpr bool stage_wide(int64_t R) {
  return R / 16 >= kStageWindow || R / 16 == kStageWindow / 2;
}

// (x * stage_recip(cpr)) >> 16 == x / cpr for every x < 2 * kStageWindow and
// 1 <= cpr < kStageWindow: the error of the scaled reciprocal stays below
// x / 65536 < 1 / cpr, too small to cross an integer.
constexpr uint32_t stage_recip(uint32_t cpr) { return 65536u / cpr + 1u; }
constexpr bool stage_recip_exact() {
  for (uint32_t cpr = 1; cpr < kStageWindow; cpr++)
    for (uint32_t x = 0; x < 2 * kStageWindow; x++)
      if (((x * stage_recip(cpr)) >> 16) != x / cpr) return false;
  return true;
}
static_assert(stage_recip_exact(), "reciprocal division of the narrow windows");
// stage_window / stage_lane's multiplier for rows of R bytes (rows shorter
// than a window need it).
constexpr uint32_t stage_recip_of(int64_t R) {
  return stage_cpr(R) < kStageWindow ? stage_recip(stage_cpr(R)) : 0u;
}

// Chunks and windows of a launch over walk rows [row_begin, row_end); the
// launcher keeps a launch at kStageMaxChunks chunks or fewer (stage_max_rows).
constexpr uint32_t stage_chunks(const XferArgs &a) {
  return (a.row_end - a.row_begin) * stage_cpr(a.R);
}
constexpr uint32_t stage_windows(const XferArgs &a) {
  return (uint32_t)(((uint64_t)stage_chunks(a) + kStageWindow - 1) / kStageWindow);
}
constexpr uint32_t stage_blocks(const XferArgs &a) {
  return (stage_windows(a) + kWavesPerBlock - 1) / kWavesPerBlock;
}
constexpr uint32_t stage_max_rows(int64_t R) { return kStageMaxChunks / stage_cpr(R); }

// The piece of a launch over walk rows [a.row_begin, a.row_end) that starts at
// walk row r and holds at most `step` rows; its staging rows start where row r
// sits in the whole launch's staging buffer.
constexpr XferArgs stage_piece(const XferArgs &a, uint32_t r, uint32_t step) {
  XferArgs p = a;
  p.row_begin = r;
  p.row_end = a.row_end - r > step ? r + step : a.row_end;
  p.host = a.host + (int64_t)(r - a.row_begin) * a.R;
  return p;
}

// Window w of a launch: its first chunk c0, the row ra (relative to
// row_begin) and chunk ka of that chunk, and the rows it touches; recip =
// stage_recip_of(R). One division per window: the window's
// last row follows from ka + 63 < 2 * max(cpr, kStageWindow) by a comparison
// (wide) or the reciprocal (narrow).
struct StageWindow {
  uint32_t c0, ra, ka, rows;
};

constexpr StageWindow stage_window(const XferArgs &a, uint32_t w, uint32_t recip) {
  const uint32_t cpr = stage_cpr(a.R);
  StageWindow s{w * kStageWindow, 0, 0, 0};
  s.ra = s.c0 / cpr;
  s.ka = s.c0 - s.ra * cpr;
  const uint32_t x = s.ka + kStageWindow - 1;
  const uint32_t last = cpr >= kStageWindow ? (x >= cpr ? 1u : 0u) : (x * recip) >> 16;
  s.rows = umin(last + 1, (a.row_end - a.row_begin) - s.ra);
  return s;
}

// Lane `lane` of window s moves chunk k of the window's row j (row ra + j);
// recip = stage_recip_of(R).
constexpr void stage_lane(const StageWindow &s, uint32_t cpr, uint32_t recip, uint32_t lane,
                          uint32_t &j, uint32_t &k) {
  const uint32_t x = s.ka + lane;
  j = cpr >= kStageWindow ? (x >= cpr ? 1u : 0u) : (x * recip) >> 16;
  k = x - j * cpr;
}

// A tile of the LDS variant: positions [i0, i0+nt), pairs [lcf, lcf+nl).
struct Tile {
  uint32_t i0, lcf, nt, nl;
};

constexpr Tile tile_of(const XferArgs &a, const TileArgs &ta, uint32_t block) {
  uint32_t bt = 0, bl = 0;
  if (ta.token_major) {
    bt = block / ta.tiles_lc;
    bl = block - bt * ta.tiles_lc;
  } else {
    bl = block / ta.tiles_t;
    bt = block - bl * ta.tiles_t;
  }
  Tile t{bt * ta.tile_t, bl * ta.tile_lc, 0, 0};
  t.nt = umin(ta.tile_t, a.n - t.i0);
  t.nl = umin(ta.tile_lc, a.nlc - t.lcf);
  return t;
}

// Chunk f of a tile walk -> (pair, position, chunk in row), pair-major or
// position-major.
constexpr void tile_walk(const Tile &t, uint32_t cpr, bool pos_major, uint32_t f, uint32_t &lc_t,
                         uint32_t &p_t, uint32_t &k) {
  const uint32_t row = f / cpr;
  k = f - row * cpr;
  if (pos_major) {
    p_t = row / t.nl;
    lc_t = row - p_t * t.nl;
  } else {
    lc_t = row / t.nt;
    p_t = row - lc_t * t.nt;
  }
}

// LDS chunk slot of (pair, position, chunk) inside a tile: pair-major.
constexpr uint32_t tile_slot(const Tile &t, uint32_t cpr, uint32_t lc_t, uint32_t p_t,
                             uint32_t k) {
  return (lc_t * t.nt + p_t) * cpr + k;
}

}  // namespace kvt
