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

namespace {

__device__ __forceinline__ uint8_t *dev_row(const XferArgs &a, uint32_t i, uint32_t lc) {
  return a.dev_tab[a.lc0 + lc] + a.tok[2 * i] * a.R;
}

__device__ __forceinline__ uint8_t *host_row(const XferArgs &a, uint32_t i, uint32_t lc) {
  return a.host + ((int64_t)(a.lc0 + lc) * a.lc_stride + a.tok[2 * i + 1]) * a.R;
}

}  // namespace

// Direct path: block b moves walk rows [row_begin + b*rows_per_block, ...) of
// the host-order walk; lanes take consecutive chunks of those rows.
template <bool kToHost>
__global__ __launch_bounds__(kXferThreads) void xfer_rows(XferArgs a) {
  for (uint32_t blk = blockIdx.x; blk < a.nblocks; blk += gridDim.x) {
  const uint32_t row0 = a.row_begin + blk * a.rows_per_block;
  const uint32_t nrows = min(a.rows_per_block, a.row_end - row0);
  const uint32_t nchunks = nrows * a.cpr;
  for (uint32_t base = 0; base < nchunks; base += kChunksPerBlock) {
    chunk_t v[kXferUnroll];
    chunk_t *dst[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      const uint32_t f = base + u * kXferThreads + threadIdx.x;
      dst[u] = nullptr;
      if (f < nchunks) {
        const uint32_t rr = f / a.cpr;
        const uint32_t k = f - rr * a.cpr;
        uint32_t i, lc;
        walk_row(a, row0 + rr, i, lc);
        chunk_t *d = reinterpret_cast<chunk_t *>(dev_row(a, i, lc)) + k;
        chunk_t *h = reinterpret_cast<chunk_t *>(host_row(a, i, lc)) + k;
        const chunk_t *src = kToHost ? d : h;
        dst[u] = kToHost ? h : d;
        v[u] = __builtin_nontemporal_load(src);
      }
    }
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      if (!dst[u]) continue;
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
// (a.host: walk row r at (r - row_begin) * R), the scatter unpacks them. A wave
// is K lane groups of 64/K lanes; its task is K batches of K consecutive walk
// rows. The wave steps the walk position row by row (uniform across the wave,
// so it lives in scalar registers), loads each row's device slot once, and
// hands the row's two addresses to its lane group, whose lanes move the row's
// 16-byte chunks, lane-consecutive, in passes of 64/K chunks. Each wave takes
// one task of a large grid: many small tasks keep more of HBM busy than a few
// long ones.
typedef uint32_t vec16_t __attribute__((ext_vector_type(4)));
// The same 16 bytes addressed in the global address space: the device buffers
// and the staging buffer are device memory, and naming that lets the compiler
// emit global rather than flat accesses.
typedef __attribute__((address_space(1))) vec16_t gvec16_t;

template <bool kGather, uint32_t K>
__global__ __launch_bounds__(kXferThreads) void stage_rows(
    XferArgs a, uint32_t rows_per_task, const int64_t *__restrict__ tok,
    uint8_t *const *__restrict__ dev_tab) {
  constexpr uint32_t kLanes = 64 / K;  // lanes per row
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t grp = lane / kLanes, sub = lane % kLanes;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t cpr = (uint32_t)(a.R >> 4);  // 16-byte chunks per row
  const uint32_t ntasks = (a.row_end - a.row_begin + rows_per_task - 1) / rows_per_task;
  for (uint32_t t = blockIdx.x * kWavesPerBlock + wave; t < ntasks;
       t += gridDim.x * kWavesPerBlock) {
    const uint32_t r0 = a.row_begin + t * rows_per_task;
    const uint32_t r1 = min(r0 + rows_per_task, a.row_end);
    WalkPos w = walk_at(a, r0);
    gvec16_t *dev[K];
    gvec16_t *stg[K];
#pragma unroll
    for (uint32_t u = 0; u < K; u++) {  // batch u: rows r0 + u*K + g for group g
      dev[u] = stg[u] = nullptr;
#pragma unroll
      for (uint32_t g = 0; g < K; g++) {
        const uint32_t r = r0 + u * K + g;
        if (r < r1) {
          gvec16_t *d = (gvec16_t *)(dev_tab[a.lc0 + w.lc] + tok[2 * (w.base + w.pos)] * a.R);
          gvec16_t *st = (gvec16_t *)(a.host + (int64_t)(r - a.row_begin) * a.R);
          if (grp == g) {
            dev[u] = d;
            stg[u] = st;
          }
          walk_next(a, w);
        }
      }
    }
    for (uint32_t k0 = 0; k0 < cpr; k0 += kLanes) {
      const uint32_t k = k0 + sub;
      vec16_t v[K];
#pragma unroll
      for (uint32_t u = 0; u < K; u++)
        if (dev[u] && k < cpr) v[u] = __builtin_nontemporal_load((kGather ? dev[u] : stg[u]) + k);
#pragma unroll
      for (uint32_t u = 0; u < K; u++)
        if (dev[u] && k < cpr) __builtin_nontemporal_store(v[u], (kGather ? stg[u] : dev[u]) + k);
    }
  }
}

// LDS-staged path: a workgroup owns a tile of nt positions x nl pairs. It reads
// the tile in source-address order into LDS (slot (pair, position)), then
// writes it out in destination-address order. Device order is pair-major;
// host order is position-major for page_first and pair-major otherwise.
template <bool kToHost>
__global__ __launch_bounds__(kXferThreads) void xfer_tiles_lds(XferArgs a, TileArgs ta) {
  extern __shared__ chunk_t lds[];
  for (uint32_t blk = blockIdx.x; blk < a.nblocks; blk += gridDim.x) {
  const Tile t = tile_of(a, ta, blk);
  const uint32_t cpr = a.cpr;
  const uint32_t nchunks = t.nt * t.nl * cpr;
  const bool host_pos_major = ta.token_major != 0;

  // phase 1: source -> LDS, in source order
  const bool src_pos_major = kToHost ? false : host_pos_major;
  for (uint32_t base = 0; base < nchunks; base += kChunksPerBlock) {
    chunk_t v[kXferUnroll];
    uint32_t slot[kXferUnroll];
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      const uint32_t f = base + u * kXferThreads + threadIdx.x;
      slot[u] = 0xffffffffu;
      if (f < nchunks) {
        uint32_t lc_t, p_t, k;
        tile_walk(t, cpr, src_pos_major, f, lc_t, p_t, k);
        const uint32_t i = t.i0 + p_t, lc = t.lcf + lc_t;
        const chunk_t *src = reinterpret_cast<const chunk_t *>(kToHost ? dev_row(a, i, lc)
                                                                    : host_row(a, i, lc)) + k;
        v[u] = __builtin_nontemporal_load(src);
        slot[u] = tile_slot(t, cpr, lc_t, p_t, k);
      }
    }
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++)
      if (slot[u] != 0xffffffffu) lds[slot[u]] = v[u];
  }
  __syncthreads();

  // phase 2: LDS -> destination, in destination order
  const bool dst_pos_major = kToHost ? host_pos_major : false;
  for (uint32_t base = 0; base < nchunks; base += kChunksPerBlock) {
#pragma unroll
    for (int u = 0; u < kXferUnroll; u++) {
      const uint32_t f = base + u * kXferThreads + threadIdx.x;
      if (f < nchunks) {
        uint32_t lc_t, p_t, k;
        tile_walk(t, cpr, dst_pos_major, f, lc_t, p_t, k);
        const uint32_t i = t.i0 + p_t, lc = t.lcf + lc_t;
        chunk_t *dst = reinterpret_cast<chunk_t *>(kToHost ? host_row(a, i, lc) : dev_row(a, i, lc)) + k;
        *dst = lds[tile_slot(t, cpr, lc_t, p_t, k)];
      }
    }
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

hipError_t launch_rows(const XferArgs &a, uint32_t blocks, bool to_host, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  if (to_host)
    hipLaunchKernelGGL((xfer_rows<true>), dim3(blocks), dim3(kXferThreads), 0, s, a);
  else
    hipLaunchKernelGGL((xfer_rows<false>), dim3(blocks), dim3(kXferThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stage(const XferArgs &a, uint32_t rows_per_task, uint32_t blocks, bool gather,
                        hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  const int64_t *tok = a.tok;
  uint8_t *const *tab = (uint8_t *const *)a.dev_tab;
  const dim3 grid(blocks), block(kXferThreads);
  switch (stage_lane_groups(a.R) * 2 + (gather ? 1 : 0)) {
    case 9: hipLaunchKernelGGL((stage_rows<true, 4>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
    case 8: hipLaunchKernelGGL((stage_rows<false, 4>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
    case 5: hipLaunchKernelGGL((stage_rows<true, 2>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
    case 4: hipLaunchKernelGGL((stage_rows<false, 2>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
    case 3: hipLaunchKernelGGL((stage_rows<true, 1>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
    default: hipLaunchKernelGGL((stage_rows<false, 1>), grid, block, 0, s, a, rows_per_task, tok, tab); break;
  }
  return hipGetLastError();
}

hipError_t launch_tiles_lds(const XferArgs &a, const TileArgs &t, uint32_t blocks, bool to_host,
                            hipStream_t s) {
  const size_t lds = (size_t)t.tile_t * t.tile_lc * a.R;
  if (blocks == 0) return hipSuccess;
  if (to_host)
    hipLaunchKernelGGL(xfer_tiles_lds<true>, dim3(blocks), dim3(kXferThreads), lds, s, a, t);
  else
    hipLaunchKernelGGL(xfer_tiles_lds<false>, dim3(blocks), dim3(kXferThreads), lds, s, a, t);
  return hipGetLastError();
}

}  // namespace kvt
