// kernels.hip — gfx950 kernels of the cross-tier KV transfer.
//
// Zero-copy gather/scatter between the device KV buffers (HBM) and the pinned,
// device-mapped host pool: the GPU itself loads and stores host memory over
// the host link (the "GPU-assisted I/O kernels" / "UVA copy" of the HiCache
// system design page, section "data transfer optimisation", and of the Baidu
// KV cache page, "optimisation techniques"), instead of one copy-engine
// descriptor per contiguous segment.
//
// The work is pure data movement: no arithmetic on values, no MFMA. Each lane
// moves 8-byte chunks, so one wave instruction covers 512 B of consecutive
// chunks; rows are >= 16 B and 16-B aligned on both sides, and every row is
// contiguous on both sides, so the layout transpose is row-granular and the
// accesses stay fully coalesced on both sides. Loads are non-temporal (nothing
// is re-read). Stores to the host pool are ordinary, which sustained more
// host-link bandwidth than non-temporal stores on this part; the direct load's
// stores into the device buffers are non-temporal, which leaves less to write
// back from L2 at the end of each per-layer launch (+0.2% on a 78-layer load
// of 37.7 MB layers, one launch per layer).
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace kvt {

typedef uint32_t chunk_t __attribute__((ext_vector_type(2)));
static_assert(sizeof(chunk_t) == kChunkBytes, "chunk size");
// The same 8 bytes addressed in the global address space (device buffers and
// the mapped host pool both are), so that the direct kernel's accesses are
// global rather than flat ones.
typedef __attribute__((address_space(1))) chunk_t gchunk_t;

// Where the direct kernel's slots past a block's last chunk read and write:
// one 8-byte chunk per lane of a wave, never read back by anyone.
constexpr int kSinkChunks = 64;
__device__ chunk_t g_sink[kSinkChunks];

namespace {

__device__ __forceinline__ uint8_t *dev_row(const XferArgs &a, uint32_t i, uint32_t lc) {
  return a.dev_tab[a.lc0 + lc] + a.tok[2 * i] * a.R;
}

__device__ __forceinline__ uint8_t *host_row(const XferArgs &a, uint32_t i, uint32_t lc) {
  return a.host + ((int64_t)(a.lc0 + lc) * a.lc_stride + a.tok[2 * i + 1]) * a.R;
}

// Paced kernels: a workgroup's first max(1, a.pace_burst) blocks go out at
// once (the start of a call is latency-bound); from then on each block waits
// until the device's constant-rate wall clock reaches `next`, the earliest
// start of the workgroup's next block, which then moves one interval on. A
// workgroup that fell behind keeps at most one interval of credit, so it
// cannot burst to catch up. The workgroups end their bursts together, so each
// starts its schedule at its own fraction of an interval: their blocks then
// go out evenly spread instead of all at once every interval.
__device__ __forceinline__ void pace_block(uint64_t &next, uint32_t &done, const XferArgs &a) {
  const uint32_t burst = max(1u, a.pace_burst);
  if (done < burst) {  // the last burst block starts the schedule
    if (++done == burst)
      next = (uint64_t)wall_clock64() + a.pace_ticks +
             (uint64_t)a.pace_ticks * blockIdx.x / gridDim.x;
    return;
  }
  const uint32_t ticks = a.pace_ticks;
  uint64_t now = (uint64_t)wall_clock64();
  while (now < next) {
    __builtin_amdgcn_s_sleep(4);
    now = (uint64_t)wall_clock64();
  }
  next = (now - next > ticks ? now - ticks : next) + ticks;
}

}  // namespace

// Direct path: block b moves walk rows [row_begin + b*rows_per_block, ...) of
// the host-order walk; lanes take consecutive chunks of those rows.
// kPaced: each workgroup starts its blocks at least a.pace_ticks apart on the
// device's constant-rate wall clock, so that the grid as a whole produces host
// traffic at a set rate instead of at what its workgroups can issue; a
// workgroup that fell behind may catch up by one block, no more.
// kDepth: chunks each lane keeps in flight (the slots of one pass); a block of
// rows_per_block rows takes ceil(its chunks / (256 * kDepth)) passes.
template <bool kToHost, bool kPaced, int kDepth>
__global__ __launch_bounds__(kXferThreads) void xfer_rows(XferArgs a) {
  uint64_t next = kPaced ? (uint64_t)wall_clock64() : 0;
  uint32_t done = 0;
  for (uint32_t blk = blockIdx.x; blk < a.nblocks; blk += gridDim.x) {
  if (kPaced) pace_block(next, done, a);
  const uint32_t row0 = a.row_begin + blk * a.rows_per_block;
  const uint32_t nrows = min(a.rows_per_block, a.row_end - row0);
  const uint32_t nchunks = nrows * a.cpr;
  for (uint32_t base = 0; base < nchunks; base += kXferThreads * kDepth) {
    // Branch-free slots: a slot past the block's chunks reads and writes the
    // sink instead (its index arithmetic takes the block's last chunk, so its
    // index loads stay in bounds). Then every slot's index-pair and
    // buffer-table loads issue together under one wait, the payload loads all
    // go out before any is waited for, and each store waits only for its own
    // load. Under a per-slot branch the compiler waits for every outstanding
    // access at each slot (it cannot count accesses across divergent
    // branches); loads and stores complete in issue order, so the slots' host
    // accesses would go out one at a time.
    gchunk_t *src[kDepth];
    gchunk_t *dst[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      const uint32_t f0 = base + u * kXferThreads + threadIdx.x;
      const bool live = f0 < nchunks;
      const uint32_t f = live ? f0 : nchunks - 1;
      const uint32_t rr = f / a.cpr;
      const uint32_t k = f - rr * a.cpr;
      uint32_t i, lc;
      walk_row(a, row0 + rr, i, lc);
      gchunk_t *d = (gchunk_t *)dev_row(a, i, lc) + k;
      gchunk_t *h = (gchunk_t *)host_row(a, i, lc) + k;
      gchunk_t *const sink = (gchunk_t *)(g_sink + (threadIdx.x & (kSinkChunks - 1)));
      src[u] = live ? (kToHost ? d : h) : sink;
      dst[u] = live ? (kToHost ? h : d) : sink;
    }
    chunk_t v[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; u++) v[u] = __builtin_nontemporal_load(src[u]);
#pragma unroll
    for (int u = 0; u < kDepth; u++) {
      if (!kToHost)
        __builtin_nontemporal_store(v[u], dst[u]);
      else
        *dst[u] = v[u];
    }
  }
  }
}

// Staged path, device side (HBM to HBM): kGather packs the walk rows
// [row_begin, row_end) from the device buffers into a dense staging buffer
// (a.host: walk row r at (r - row_begin) * R), the scatter unpacks them. Each
// wave moves one 1 KiB window of the staging buffer's chunk stream per
// iteration (stage_window / stage_lane): one 16-byte chunk per lane, so every
// pass is full whatever the row size, and each wave's work is short, which
// keeps more of HBM busy than long per-wave tasks do. Wide rows take their
// two possible device addresses in scalar registers (the window's position is
// uniform across the wave); narrow rows resolve one row per lane and pass the
// addresses across the wave.
typedef uint32_t vec16_t __attribute__((ext_vector_type(4)));
// The same 16 bytes addressed in the global address space: the device buffers
// and the staging buffer are device memory, and naming that lets the compiler
// emit global rather than flat accesses.
typedef __attribute__((address_space(1))) vec16_t gvec16_t;

namespace {

__device__ __forceinline__ gvec16_t *stage_row(const XferArgs &a, const WalkPos &w,
                                               const int64_t *__restrict__ tok,
                                               uint8_t *const *__restrict__ dev_tab) {
  return (gvec16_t *)(dev_tab[a.lc0 + w.lc] + tok[2 * (w.base + w.pos)] * a.R);
}

// The value `v` of lane `src` (ds_bpermute addresses lanes in bytes).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)v);
}

}  // namespace

template <bool kGather, bool kWide>
__global__ __launch_bounds__(kXferThreads) void stage_windows(
    XferArgs a, uint32_t recip, const int64_t *__restrict__ tok,
    uint8_t *const *__restrict__ dev_tab) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t cpr = stage_cpr(a.R);
  const uint32_t total = stage_chunks(a);
  const uint32_t nwin = stage_windows(a);
  gvec16_t *const stg = (gvec16_t *)a.host;
  for (uint32_t w = blockIdx.x * kWavesPerBlock + wave; w < nwin;
       w += gridDim.x * kWavesPerBlock) {
    const StageWindow s = stage_window(a, w, recip);
    gvec16_t *d = nullptr;
    if (kWide) {
      // stage_lane's mapping with the per-lane part reduced to a compare: the
      // lanes below split = cpr - ka move chunk ka + lane of the first row,
      // the others chunk lane - split of the second
      WalkPos wp = walk_at(a, a.row_begin + s.ra);
      gvec16_t *const first = stage_row(a, wp, tok, dev_tab);
      gvec16_t *second = first;
      if (s.rows > 1) {
        walk_next(a, wp);
        second = stage_row(a, wp, tok, dev_tab);
      }
      const uint32_t split = cpr - s.ka;
      d = (lane < split ? first + s.ka : second - split) + lane;
    } else {
      uint32_t j = 0, k = 0;
      stage_lane(s, cpr, recip, lane, j, k);
      uint64_t mine = 0;
      if (lane < s.rows) {
        const WalkPos wp = walk_at(a, a.row_begin + s.ra + lane);
        mine = (uint64_t)stage_row(a, wp, tok, dev_tab);
      }
      d = (gvec16_t *)((uint64_t)lane_value((uint32_t)mine, j) |
                       ((uint64_t)lane_value((uint32_t)(mine >> 32), j) << 32)) + k;
    }
    const uint32_t c = s.c0 + lane;
    if (c < total) {
      gvec16_t *const st = stg + c;
      const vec16_t v = __builtin_nontemporal_load(kGather ? d : st);
      __builtin_nontemporal_store(v, kGather ? st : d);
    }
  }
}

// LDS-staged path: a workgroup owns a tile of nt positions x nl pairs. It reads
// the tile in source-address order into LDS (slot (pair, position)), then
// writes it out in destination-address order. Device order is pair-major;
// host order is position-major for page_first and pair-major otherwise.
// kPaced: as xfer_rows, one interval per tile.
template <bool kToHost, bool kPaced>
__global__ __launch_bounds__(kXferThreads) void xfer_tiles_lds(XferArgs a, TileArgs ta) {
  extern __shared__ chunk_t lds[];
  uint64_t next = kPaced ? (uint64_t)wall_clock64() : 0;
  uint32_t done = 0;
  for (uint32_t blk = blockIdx.x; blk < a.nblocks; blk += gridDim.x) {
  if (kPaced) pace_block(next, done, a);
  const Tile t = tile_of(a, ta, blk);
  const uint32_t cpr = a.cpr;
  const uint32_t nchunks = t.nt * t.nl * cpr;
  const bool host_pos_major = ta.token_major != 0;

  // phase 1: source -> LDS, in source order. As in xfer_rows the slots are
  // branch-free up to the LDS writes (a slot past the tile's chunks loads the
  // sink), so the source loads are all in flight at once.
  const bool src_pos_major = kToHost ? false : host_pos_major;
  for (uint32_t base = 0; base < nchunks; base += kChunksPerBlock) {
    gchunk_t *src[kXferUnroll];
    uint32_t slot[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      const uint32_t f0 = base + u * kXferThreads + threadIdx.x;
      const bool live = f0 < nchunks;
      uint32_t lc_t, p_t, k;
      tile_walk(t, cpr, src_pos_major, live ? f0 : nchunks - 1, lc_t, p_t, k);
      const uint32_t i = t.i0 + p_t, lc = t.lcf + lc_t;
      gchunk_t *const s0 = (gchunk_t *)(kToHost ? dev_row(a, i, lc) : host_row(a, i, lc)) + k;
      src[u] = live ? s0 : (gchunk_t *)(g_sink + (threadIdx.x & (kSinkChunks - 1)));
      slot[u] = live ? tile_slot(t, cpr, lc_t, p_t, k) : 0xffffffffu;
    }
    chunk_t v[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) v[u] = __builtin_nontemporal_load(src[u]);
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++)
      if (slot[u] != 0xffffffffu) lds[slot[u]] = v[u];
  }
  __syncthreads();

  // phase 2: LDS -> destination, in destination order; a slot past the
  // tile's chunks reads the tile's last chunk and writes it to the sink.
  const bool dst_pos_major = kToHost ? host_pos_major : false;
  for (uint32_t base = 0; base < nchunks; base += kChunksPerBlock) {
    gchunk_t *dst[kXferUnroll];
    uint32_t slot[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      const uint32_t f0 = base + u * kXferThreads + threadIdx.x;
      const bool live = f0 < nchunks;
      uint32_t lc_t, p_t, k;
      tile_walk(t, cpr, dst_pos_major, live ? f0 : nchunks - 1, lc_t, p_t, k);
      const uint32_t i = t.i0 + p_t, lc = t.lcf + lc_t;
      gchunk_t *const d0 = (gchunk_t *)(kToHost ? host_row(a, i, lc) : dev_row(a, i, lc)) + k;
      dst[u] = live ? d0 : (gchunk_t *)(g_sink + (threadIdx.x & (kSinkChunks - 1)));
      slot[u] = tile_slot(t, cpr, lc_t, p_t, k);
    }
    chunk_t v[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) v[u] = lds[slot[u]];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) *dst[u] = v[u];
  }
  __syncthreads();  // the next tile reuses the LDS
  }
}

// Index pairs of a request from its raw index arrays, on the device:
// tok[2i] = dev_idx[i], tok[2i+1] = the host key of host_idx[i] in the pool's
// layout (layer_first h; page_first h*L*C; page_first_direct
// (h/ps)*L*C*ps + h%ps), as the host-side staging writes them.
__global__ __launch_bounds__(kXferThreads) void pack_pairs(const int64_t *__restrict__ dev_idx,
                                                           const int64_t *__restrict__ host_idx,
                                                           int64_t *__restrict__ tok, uint32_t n,
                                                           int32_t layout, int64_t lc, int32_t ps) {
  const uint32_t i = blockIdx.x * kXferThreads + threadIdx.x;
  if (i >= n) return;
  const int64_t h = host_idx[i];
  int64_t key = h;
  if (layout == kLayoutPageFirst) {
    key = h * lc;
  } else if (layout == kLayoutPageFirstDirect) {
    const int64_t q = h / ps;
    key = q * lc * ps + (h - q * ps);
  }
  tok[2 * i] = dev_idx[i];
  tok[2 * i + 1] = key;
}

hipError_t launch_pack_pairs(const int64_t *dev_idx, const int64_t *host_idx, int64_t *tok,
                             uint32_t n, int32_t layout, int64_t lc, int32_t ps, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_pairs, dim3((n + kXferThreads - 1) / kXferThreads), dim3(kXferThreads),
                     0, s, dev_idx, host_idx, tok, n, layout, lc, ps);
  return hipGetLastError();
}

namespace {

template <int kDepth>
void launch_rows_depth(const XferArgs &a, dim3 grid, bool to_host, size_t lds_bytes,
                       hipStream_t s) {
  const dim3 block(kXferThreads);
  switch ((a.pace_ticks ? 2 : 0) + (to_host ? 1 : 0)) {
    case 3: hipLaunchKernelGGL((xfer_rows<true, true, kDepth>), grid, block, lds_bytes, s, a); break;
    case 2: hipLaunchKernelGGL((xfer_rows<false, true, kDepth>), grid, block, lds_bytes, s, a); break;
    case 1: hipLaunchKernelGGL((xfer_rows<true, false, kDepth>), grid, block, lds_bytes, s, a); break;
    default: hipLaunchKernelGGL((xfer_rows<false, false, kDepth>), grid, block, lds_bytes, s, a); break;
  }
}

}  // namespace

hipError_t launch_rows(const XferArgs &a, uint32_t blocks, bool to_host, size_t lds_bytes,
                       int depth, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks);
  switch (depth) {
    case 1: launch_rows_depth<1>(a, grid, to_host, lds_bytes, s); break;
    case 2: launch_rows_depth<2>(a, grid, to_host, lds_bytes, s); break;
    case 4: launch_rows_depth<4>(a, grid, to_host, lds_bytes, s); break;
    case 8: launch_rows_depth<8>(a, grid, to_host, lds_bytes, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stage(const XferArgs &a, uint32_t cap, bool gather, hipStream_t s,
                        uint32_t *launches, uint32_t *last_grid) {
  const int64_t *tok = a.tok;
  uint8_t *const *tab = (uint8_t *const *)a.dev_tab;
  const uint32_t recip = stage_recip_of(a.R);
  const uint32_t step = stage_max_rows(a.R);
  const dim3 block(kXferThreads);
  for (uint32_t r = a.row_begin; r < a.row_end; r += step) {
    const XferArgs p = stage_piece(a, r, step);
    const dim3 grid(grid_for(stage_blocks(p), cap));
    switch ((stage_wide(a.R) ? 2 : 0) + (gather ? 1 : 0)) {
      case 3: hipLaunchKernelGGL((stage_windows<true, true>), grid, block, 0, s, p, recip, tok, tab); break;
      case 2: hipLaunchKernelGGL((stage_windows<false, true>), grid, block, 0, s, p, recip, tok, tab); break;
      case 1: hipLaunchKernelGGL((stage_windows<true, false>), grid, block, 0, s, p, recip, tok, tab); break;
      default: hipLaunchKernelGGL((stage_windows<false, false>), grid, block, 0, s, p, recip, tok, tab); break;
    }
    if (launches) (*launches)++;
    if (last_grid) *last_grid = grid.x;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_tiles_lds(const XferArgs &a, const TileArgs &t, uint32_t blocks, bool to_host,
                            hipStream_t s) {
  const size_t lds = (size_t)t.tile_t * t.tile_lc * a.R;
  if (blocks == 0) return hipSuccess;
  const dim3 grid(blocks), block(kXferThreads);
  switch ((a.pace_ticks ? 2 : 0) + (to_host ? 1 : 0)) {
    case 3: hipLaunchKernelGGL((xfer_tiles_lds<true, true>), grid, block, lds, s, a, t); break;
    case 2: hipLaunchKernelGGL((xfer_tiles_lds<false, true>), grid, block, lds, s, a, t); break;
    case 1: hipLaunchKernelGGL((xfer_tiles_lds<true, false>), grid, block, lds, s, a, t); break;
    default: hipLaunchKernelGGL((xfer_tiles_lds<false, false>), grid, block, lds, s, a, t); break;
  }
  return hipGetLastError();
}

}  // namespace kvt
