// kernels.hpp — launch interface of the gfx950 transfer kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "xfer_walk.hpp"

namespace kvt {

// `blocks` is the number of workgroups to launch; the kernels stride over
// a.nblocks blocks of work (plan_rows / plan_tiles), so blocks may be smaller.
// lds_bytes: dynamic LDS asked for per workgroup (the kernel uses none; a
// compute unit's whole LDS keeps other kernels' workgroups off its compute unit).
// depth: chunks each lane keeps in flight, 1, 2, 4 or 8 (else hipErrorInvalidValue).
hipError_t launch_rows(const XferArgs &a, uint32_t blocks, bool to_host, size_t lds_bytes,
                       int depth, hipStream_t s);
// The staged path's device-side pass over walk rows [a.row_begin, a.row_end):
// gather packs them from the device buffers into the staging buffer a.host,
// the scatter unpacks them. One launch per stage_max_rows(R) rows (one for any
// staging chunk of 32 GiB or less), each on at most `cap` workgroups (0 = one
// per kWavesPerBlock windows): the waves stride over the windows. Adds the
// launches made to *launches and sets *last_grid to the last launch's grid
// (either may be null). An empty range launches nothing.
hipError_t launch_stage(const XferArgs &a, uint32_t cap, bool gather, hipStream_t s,
                        uint32_t *launches, uint32_t *last_grid);
// The index pairs {device slot, host key} of n positions from the raw index
// arrays (all three device pointers): lc = L*C of the pool.
hipError_t launch_pack_pairs(const int64_t *dev_idx, const int64_t *host_idx, int64_t *tok,
                             uint32_t n, int32_t layout, int64_t lc, int32_t ps, hipStream_t s);
hipError_t launch_tiles_lds(const XferArgs &a, const TileArgs &t, uint32_t blocks, bool to_host,
                            hipStream_t s);

}  // namespace kvt
