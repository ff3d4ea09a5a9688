// kernels.hpp — launch interface of the gfx950 transfer kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "xfer_walk.hpp"

namespace kvt {

// `blocks` is the number of workgroups to launch; the kernels stride over
// a.nblocks blocks of work (plan_rows / plan_tiles), so blocks may be smaller.
// dense: the host side of a is a device staging buffer (staged path).
hipError_t launch_rows(const XferArgs &a, uint32_t blocks, bool to_host, bool dense,
                       hipStream_t s);
hipError_t launch_tiles_lds(const XferArgs &a, const TileArgs &t, uint32_t blocks, bool to_host,
                            hipStream_t s);

}  // namespace kvt
