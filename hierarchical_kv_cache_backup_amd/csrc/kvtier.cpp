// kvtier.cpp — C ABI of the cross-tier KV transfer: pool lifetime, request
// intake, path selection, the kernel and copy-engine executors, per-layer load
// events, statistics and error reporting.
//
// Submission model (Kunlunxin tuning page, section 2.2; Baidu KV cache page,
// "bidirectional async transfer"): a call validates, plans and ENQUEUES on the
// caller's stream, then returns; backup and load have separate state and locks
// so one thread per direction can submit concurrently on private streams.
#include <hip/hip_runtime.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "kvtier.h"
#include "plan.hpp"

namespace kvt {

thread_local std::string g_err;
void set_error(const std::string &msg) { g_err = msg; }

namespace {

constexpr int kStagingSlots = 16;  // index-staging buffers in flight per direction
constexpr int64_t kMaxRowsPerLaunch = (int64_t)1 << 31;
constexpr double kExtentPlanLimit = 4.0 * 1024 * 1024;  // staged extents AUTO lists exactly
// Staged path: chunks ramp (chunk_plan) on halves of at least
// staged_chunk_bytes / kRampMinDiv; below that the pass the ramp shortens is
// shorter than the launches and copies it adds.
constexpr double kRampMinDiv = 16.0;
// A paced kernel grid delivers slightly less than its pace: 99.2% alone (2.9 GB
// write-back paced to 55.9 GB/s), 97.9-98.1% beside an HBM-bound kernel
// (paced to 55-57 GB/s); the model takes 99%.
constexpr double kPaceYield = 0.99;

int fail(int code, const std::string &msg) {
  set_error(msg);
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(KV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Runs an entry point's body so that no C++ exception crosses the C ABI: an
// allocation failure of the library's own host bookkeeping becomes KV_ENOMEM.
template <typename F>
int guarded(const char *what, F &&body) {
  try {
    return body();
  } catch (const std::bad_alloc &) {
    return fail(KV_ENOMEM, std::string(what) + ": out of host memory");
  } catch (const std::exception &ex) {
    return fail(KV_EINVAL, std::string(what) + ": " + ex.what());
  }
}

struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) {
      err = hipSetDevice(dev);
      changed = err == hipSuccess;
    }
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

// Pinned host + device copy of the per-position {device slot, host key} pairs.
// The pinned buffer is also mapped for the device (pinned_dev), so the kernels
// can read small index arrays from it directly, without the device copy.
struct Staging {
  int64_t *pinned = nullptr;
  int64_t *pinned_dev = nullptr;
  int64_t *dev = nullptr;
  int64_t cap = 0;  // positions
  hipEvent_t ev = nullptr;
  bool pending = false;
};

struct DirState {
  std::mutex mu;
  UniqueScratch uniq;
  std::vector<Run> runs;
  std::vector<Copy> copies;
  Staging slots[kStagingSlots];
  int used = 0;  // slots opened so far
  int next = 0;  // where the search for a free slot starts
  hipEvent_t done = nullptr;  // recorded at the end of every call of this direction
  bool done_pending = false;
  std::atomic<bool> done_recorded{false};  // read without the lock by the other direction
  std::atomic<hipStream_t> done_stream{nullptr};  // the stream `done` was recorded on
  // staged path: two device staging halves (dense images of walk rows), an
  // auxiliary stream for the gather/scatter kernels, and the events that pass
  // each half between the copies (caller's stream) and the kernels (aux).
  std::vector<Extent> extents;
  std::vector<int64_t> host_run_start;  // staged path: runs of host-consecutive positions
  std::vector<int64_t> chunk_len;       // staged path: the unit's chunk lengths (rows)
  uint8_t *stage = nullptr;      // 2 * stage_cap bytes
  int64_t stage_cap = 0;         // bytes per half
  int64_t stage_use = 0;         // bytes per half the current call fills (<= stage_cap)
  hipEvent_t stage_ev = nullptr;  // the call's last use of the halves (on the caller's stream)
  bool stage_pending = false;
  hipStream_t stage_stream = nullptr;
  hipStream_t aux = nullptr;
  hipEvent_t ev_start = nullptr, ev_ready[2] = {nullptr, nullptr}, ev_free[2] = {nullptr, nullptr};

  bool free_recorded[2] = {false, false};
  uint32_t next_half = 0;  // halves alternate across chunks, groups and calls
  int last_half = -1;      // half of the latest chunk
  std::atomic<int32_t> last_path{-1};
  int64_t calls = 0, bytes = 0, launches = 0, dma = 0, last_workgroups = 0;
  double submit_us = 0, blocked_us = 0;
};

// The pinned host pool, owned jointly by the pools of a group that share it
// (kv_pool_create_shared): freed with the last of them. The writer (the pool
// kv_pool_create made) records `written` after each of its backups; a sharing
// pool's backup makes its stream wait for that event.
struct HostShare {
  int device = 0;               // the writer's device (the event lives there)
  uint8_t *host = nullptr;      // CPU address
  int64_t bytes = 0;
  bool check = false;           // KV_F_SHARE_CHECK on the writer
  std::mutex mu;
  hipEvent_t written = nullptr;
  bool recorded = false;        // the writer has backed up at least once
  uint64_t digest = 0;          // of the writer's latest backup (host slots, layer range)
  ~HostShare();
};

}  // namespace
}  // namespace kvt

using namespace kvt;

struct kv_pool {
  Geom g;
  int device = 0;
  uint32_t flags = 0;
  int32_t numa = -1;
  std::vector<uint8_t *> bufs;      // L*C device buffer bases
  uint8_t **dev_tab = nullptr;      // device copy of bufs
  uint8_t *host = nullptr;          // host pool, CPU address
  uint8_t *host_dev = nullptr;      // host pool, device-visible address
  int64_t host_bytes = 0;
  std::shared_ptr<HostShare> share; // the host pool and the group's write event
  bool reader = false;              // shares another pool's host pool; its backups move nothing
  // Landed events of kv_load. Layers are loaded in groups (one launch or one
  // batch of copies per group) and one event is recorded per group;
  // layer_src[l] names the event that covers layer l in the most recent load
  // that covered it (-1: none yet). The events form a fixed set of 2L + 16
  // made at pool creation (kv_load_layer indexes it without a lock); ev_refs
  // counts the layers naming each, and an event is recorded again only when no
  // layer names it and its last recording has completed (mark_landed), so a
  // layer's wait never moves to another load's work. ev_refs, ev_recorded and
  // ev_next are guarded by the load direction's lock.
  std::vector<hipEvent_t> layer_ev;
  std::vector<std::atomic<int32_t>> layer_src;
  std::vector<int32_t> ev_refs;
  std::vector<uint8_t> ev_recorded;
  size_t ev_next = 0;
  DirState dir[2];
  std::atomic<int32_t> path[2] = {{KV_PATH_AUTO}, {KV_PATH_AUTO}};  // per direction
  std::mutex calib_mu;
  kv_calib_t calib{};
  int wall_khz = 0;  // the device's constant wall-clock rate (paced kernels)
  int lds_max = 0;   // LDS bytes one workgroup may ask for (a compute unit's whole LDS)
  explicit kv_pool(int L) : layer_src(L) {
    for (auto &x : layer_src) x.store(-1);
  }
};

namespace kvt {
namespace {

// Defaults measured on an MI355X (PCIe Gen5 x16 host link) with 1152-byte
// rows: fixed cost per kernel call (launch, index staging, ramp) ~30 us and per
// copy-engine call ~9.5 us, both from requests of 64..32768 tokens x 78 layers;
// ~7 us between back-to-back per-layer launches of one load (kernel trace
// against event time); sustained rates at 2.9 GB per call. bench.py re-fits
// the rates live.
void default_calibration(kv_calib_t *c) {
  // A load's launches: 25 us for the first, 8.9 us for each further layer
  // group (the 7 us gap between launches and 1.9 us of the link draining and
  // ramping), at 57.3 GB/s: least squares on relative error over full-grid
  // loads of 64 to 32768 tokens x 78 layers of 1152 bytes in the three
  // layouts (1 to 78 launches), all within 2%. Backups are one launch.
  c->kernel_launch_us[0] = 30.0;
  c->kernel_launch_us[1] = 25.0;
  c->kernel_group_us[0] = c->kernel_group_us[1] = 7.0;
  c->kernel_link_gap_us[0] = 0.0;
  c->kernel_link_gap_us[1] = 1.9;
  // The staged path also takes HBM bandwidth, compute units and a second
  // stream: beside an HBM-bound kernel a staged write-back slowed it 1.16x,
  // the copy engines 1.10-1.12x. Its time model is within ~1% of measured
  // calls (4096-32768 tokens), so a 2% margin keeps it off ties and still
  // takes it where it is 3-6% faster (page-major write-backs of 8K+ tokens).
  c->staged_min_gain = 0.02;
  c->kernel_gbps[0] = 55.9;  // full grid; a capped grid is modelled per workgroup below
  c->kernel_gbps[1] = 57.3;
  // What W workgroups move on a capped grid. A workgroup keeps
  // kernel_lane_depth chunks of 8 bytes in flight per lane: a write-back
  // workgroup moves ~3.3 GB/s at the default depth of 2 (6.6 at 8), a load's
  // 3.6-4.0 at 8 (4-16 workgroups). Write-backs on the default grid (18
  // workgroups, depth 2, paced to 54 GB/s), 64 to 32768 tokens of the 78 x
  // 1152-byte MLA latent (5.8 MB to 2.9 GB) in the three layouts, fit a slow
  // start: the first ~30 MB of a call cost up to 275 us more (64-token calls
  // run at 34 GB/s, 32K-token ones at 53.6); within 4% from 512 tokens up and
  // 9.5% below (the paths there are far apart). At depth 2 the walk's jumps
  // between device rows (page_first) cost nothing measurable.
  c->kernel_wg_gbps[0] = 3.3;
  c->kernel_wg_gbps[1] = 3.8;
  c->kernel_wg_row_ns[0] = 0.0;
  c->kernel_wg_row_ns[1] = 0.0;
  c->kernel_wg_jump_ns[0] = 0.0;
  c->kernel_wg_jump_ns[1] = 0.0;
  c->kernel_wg_start_bytes[0] = 30e6;
  c->kernel_wg_start_us[0] = 275.0;
  c->kernel_wg_start_bytes[1] = 0.0;
  c->kernel_wg_start_us[1] = 0.0;
  c->dma_copy_us[0] = c->dma_copy_us[1] = 9.5;
  c->dma_gbps[0] = 56.9;  // fitted on the 2.9 GB headline call, as bench.py does
  c->dma_gbps[1] = 56.9;
  c->load_split_min_bytes = 16.0 * 1024 * 1024;
  // A write-back kernel on a full grid keeps the link full with posted host
  // writes, and an HBM-bound kernel running beside it (the model's next
  // prefill or decode) then ran ~26-46x longer (fp8 write-backs beside a
  // stream of 2 x 256 MiB reductions). Unpaced, a grid whose writes outrun
  // what the link drains (~56-57 GB/s) backs up in the memory system and the
  // write-back falls to ~39-44 GB/s (depth 2: from 18 workgroups; depth 8:
  // from 10). Paced (kernel_pace_gbps) a grid cannot outrun the link, and the
  // neighbour's cost follows the workgroups and the accesses each keeps in
  // flight (paced to 54-56 GB/s, depth 2: 16 workgroups 1.13x, 18 1.16x, 20
  // 1.19x, 24 1.28-1.30x; depth 8: 8 1.19-1.20x, 9 1.22x, 10 1.27-1.28x, 12
  // 1.43-1.48x; depth 1: 32 1.25-1.28x, 36 1.33-1.35x; depth 4: 10 1.18x;
  // the copy engines 1.11x). 18 workgroups at depth 2 are the
  // smallest grid that produces more than its pace: 53.0 GB/s beside the
  // neighbour paced to 54, 54.9 paced to 56. On the host whose link drained
  // least (1 GiB D2H copy 56.2 GB/s) a pace of 56 sagged to 52.2-52.9 GB/s on
  // 8K-32K-token write-backs and one of 55.1 held 54.6: the default pace, 54,
  // stays ~2% under that. A caller that measures its link paces at ~0.98 of
  // its D2H copy rate. The start of a call is latency-bound: 32 blocks of
  // burst per workgroup before the pacing starts keep small calls at the
  // unpaced rate. Loads keep the full grid: a load beside compute is
  // KV_F_LOAD_OVERLAP's case.
  c->kernel_max_workgroups[0] = 18;
  c->kernel_max_workgroups[1] = 0;
  c->kernel_pace_gbps[0] = 54.0;
  c->kernel_pace_gbps[1] = 0.0;
  c->kernel_pace_burst_blocks[0] = 32.0;
  c->kernel_pace_burst_blocks[1] = 0.0;
  // A capped load's workgroups each take a compute unit of their own: beside
  // the reductions below, 16 load workgroups slowed them 1.23x that way and
  // 1.43x sharing compute units with them (24: 1.28x against 1.56x). A
  // write-back's did not gain (18 workgroups at depth 2, paced: 1.34x alone on
  // their compute units, 1.17x sharing them).
  c->kernel_cu_exclusive[0] = 0.0;
  c->kernel_cu_exclusive[1] = 1.0;
  c->kernel_lane_depth[0] = 2.0;
  c->kernel_lane_depth[1] = 8.0;
  // Measured on MI355X with a streamed 24-layer load (256 MiB per layer) and an
  // HBM-bound consumer (torch int64 sums) overlapped layer by layer: the
  // consumer's slowdown beside the kernel path grows with the load's grid
  // (workgroups on compute units of their own: 8 1.17x at 29 GB/s, 16 1.23x
  // at 52.9, 24 1.28x at 56.5, 32 1.32x, 48 1.40x; a full grid 1.93x); beside
  // the copy path it is 1.14x at 56.8 GB/s. 24 workgroups is the smallest grid
  // that keeps the link full.
  c->overlap_kernel_penalty = 0.28;
  c->overlap_dma_penalty = 0.15;
  c->overlap_kernel_max_workgroups = 24;
  // On the mixed batch (load 51.2 GB || write-back 11.6 GB) with the duplex
  // caps below, the load's kernel held 56.5-56.8 GB/s (57.3 alone) beside a
  // write-back kernel of 23-24 GB/s (26.6-26.8 alone on its duplex cap of 8
  // workgroups at depth 2): 98.6-99.2% of the duplex bound, against 80% with
  // the caps off (the load on a full grid). The write-back's cap already sets
  // its rate; what the load's traffic costs it on top is charged here.
  c->duplex_kernel_penalty[0] = 0.1;
  c->duplex_kernel_penalty[1] = 0.0;
  c->duplex_kernel_max_workgroups[0] = 8;
  c->duplex_kernel_max_workgroups[1] = 32;
  c->staged_chunk_bytes = 256.0 * 1024 * 1024;
  // the device-side gather / scatter of a staged chunk (stage_windows, HBM to
  // HBM, full grid), payload rate: the 2.94 GB prefix of 1152-byte rows packs
  // in ~0.97 ms and unpacks in ~0.94 ms (6.1-6.3 TB/s of HBM traffic), so a
  // 256 MiB half takes ~88 us
  c->staged_gather_gbps = 3000.0;
  // Reading the index pairs from mapped pinned memory instead of copying them
  // first measured +0.6..1.6% at 64 tokens, even at 256, and down to -2% for
  // loads of 1K tokens and more (the reads share the link and lengthen each
  // block's dependent load chain): on for requests of at most 128 positions.
  c->index_zero_copy_max_bytes[0] = c->index_zero_copy_max_bytes[1] = 2048.0;
}

// Sets the calling thread's memory policy (Linux set_mempolicy: kMpolBind to
// the nodes of `mask`, or kMpolInterleave page by page across them), returning
// the previous policy in *old_mode / *old_mask so it can be restored. Node
// masks are one unsigned long: nodes 0..63.
constexpr int kMpolDefault = 0, kMpolBind = 2, kMpolInterleave = 3;
constexpr int kMaxNumaNodes = 8 * sizeof(unsigned long);
bool set_thread_policy(int mode, unsigned long mask, int *old_mode, unsigned long *old_mask) {
  *old_mode = kMpolDefault;
  *old_mask = 0;
  if (syscall(SYS_get_mempolicy, old_mode, old_mask, 8 * sizeof(unsigned long), nullptr, 0) != 0)
    return false;
  return syscall(SYS_set_mempolicy, mode, &mask, 8 * sizeof(unsigned long)) == 0;
}

void restore_thread_policy(int mode, unsigned long mask) {
  syscall(SYS_set_mempolicy, mode, mode == kMpolDefault ? nullptr : &mask,
          8 * sizeof(unsigned long));
}

bool numa_node_exists(int node) {
  if (node < 0 || node >= kMaxNumaNodes) return false;
  char path[96];
  std::snprintf(path, sizeof path, "/sys/devices/system/node/node%d", node);
  return access(path, F_OK) == 0;
}

// Mask of the online NUMA nodes below kMaxNumaNodes, from the kernel's list
// ("0", "0-3", "0-1,4"); 0 if it cannot be read.
unsigned long online_numa_nodes() {
  FILE *f = std::fopen("/sys/devices/system/node/online", "r");
  if (!f) return 0;
  char buf[256] = {0};
  const size_t got = std::fread(buf, 1, sizeof buf - 1, f);
  std::fclose(f);
  buf[got] = 0;
  unsigned long mask = 0;
  const char *c = buf;
  while (*c >= '0' && *c <= '9') {
    char *end = nullptr;
    long a = std::strtol(c, &end, 10), b = a;
    c = end;
    if (*c == '-') {
      b = std::strtol(c + 1, &end, 10);
      c = end;
    }
    for (long k = a; k <= b && k < kMaxNumaNodes; k++) mask |= 1ul << k;
    if (*c == ',') c++;
  }
  return mask;
}

double now_us() {
  return std::chrono::duration<double, std::micro>(
             std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

HostShare::~HostShare() {
  DeviceGuard dg(device);
  if (written) (void)hipEventDestroy(written);
  if (host) (void)hipHostFree(host);
}

// 64-bit FNV-1a over a backup request's host slots and layer range: the
// fingerprint two ranks of a group compare to confirm they name the same host
// rows (KV_F_SHARE_CHECK).
uint64_t request_digest(const int64_t *host_idx, int64_t n, int32_t l0, int32_t l1) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&h](uint64_t v, int bytes) {
    for (int b = 0; b < bytes; b++) {
      h ^= (v >> (8 * b)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  };
  mix((uint64_t)(uint32_t)l0, 4);
  mix((uint64_t)(uint32_t)l1, 4);
  for (int64_t i = 0; i < n; i++) mix((uint64_t)host_idx[i], 8);
  return h;
}

void free_staging(Staging &s) {
  if (s.pinned) (void)hipHostFree(s.pinned);
  if (s.dev) (void)hipFree(s.dev);
  s.pinned = nullptr;
  s.pinned_dev = nullptr;
  s.dev = nullptr;
  s.cap = 0;
}

// Waits for every enqueued use of the direction's staging buffers.
hipError_t drain_direction(DirState &d) {
  hipError_t first = hipSuccess;
  for (Staging &s : d.slots) {
    if (s.pending) {
      hipError_t e = hipEventSynchronize(s.ev);
      if (e != hipSuccess && first == hipSuccess) first = e;
      s.pending = false;
    }
  }
  if (d.done_pending) {
    hipError_t e = hipEventSynchronize(d.done);
    if (e != hipSuccess && first == hipSuccess) first = e;
    d.done_pending = false;
  }
  if (d.stage_pending) {
    hipError_t e = hipEventSynchronize(d.stage_ev);
    if (e != hipSuccess && first == hipSuccess) first = e;
    d.stage_pending = false;
  }
  return first;
}

// A staging slot with room for n positions. Prefers a slot whose previous
// use has completed (no wait); opens a new slot while fewer than
// kStagingSlots exist; only when every slot still carries work in flight does
// it wait for the oldest (back-pressure), adding the wait to *blocked_us.
int acquire_staging(DirState &d, int64_t n, Staging **out, double *blocked_us) {
  Staging *pick = nullptr;
  for (int k = 0; k < d.used && !pick; k++) {
    Staging &s = d.slots[(d.next + k) % d.used];
    if (!s.pending) {
      pick = &s;
    } else {
      hipError_t q = hipEventQuery(s.ev);
      if (q == hipSuccess) {
        s.pending = false;
        pick = &s;
      } else if (q != hipErrorNotReady) {
        return hip_fail(q, "index staging event");
      }
    }
  }
  if (!pick && d.used < kStagingSlots) pick = &d.slots[d.used++];
  if (!pick) {
    Staging &s = d.slots[d.next % d.used];
    const double t0 = now_us();
    hipError_t e = hipEventSynchronize(s.ev);
    *blocked_us += now_us() - t0;
    s.pending = false;
    if (e != hipSuccess) return hip_fail(e, "waiting for an index staging buffer");
    pick = &s;
  }
  d.next = (int)(pick - d.slots) + 1;
  Staging &s = *pick;
  if (s.cap < n) {
    free_staging(s);
    int64_t cap = 1024;
    while (cap < n) cap *= 2;
    hipError_t e = hipHostMalloc((void **)&s.pinned, (size_t)cap * 16,
                                 hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
      s.pinned = nullptr;
      return fail(KV_ENOMEM, "hipHostMalloc of index staging failed");
    }
    e = hipHostGetDevicePointer((void **)&s.pinned_dev, s.pinned, 0);
    if (e != hipSuccess) {
      free_staging(s);
      return hip_fail(e, "mapping the index staging buffer");
    }
    e = hipMalloc((void **)&s.dev, (size_t)cap * 16);
    if (e != hipSuccess) {
      s.dev = nullptr;
      free_staging(s);
      return fail(KV_ENOMEM, "hipMalloc of index staging failed");
    }
    s.cap = cap;
  }
  *out = &s;
  return KV_OK;
}

// ---- copy-engine executor ------------------------------------------------

// Issues copy c of (layer, component) buffer lc; adds the copy-engine calls
// made to *calls. A 2-D call goes out only over the lines whose whole
// pitch x lines region lies inside the host pool and the device buffer
// (copy_region_lines); a line left over goes out as a 1-D call.
hipError_t issue_copy(kv_pool *p, int dir, int32_t lc, const Copy &c, hipStream_t s,
                      int64_t *calls) {
  const Geom &g = p->g;
  uint8_t *dev = p->bufs[lc] + c.dev0 * g.R;
  uint8_t *host = p->host + ((int64_t)lc * g.lc_stride + c.key0) * g.R;
  const size_t width = (size_t)(c.len * g.R);
  const size_t dpitch = (size_t)(c.dev_pitch * g.R), hpitch = (size_t)(c.key_pitch * g.R);
  auto lines_1d = [&](int64_t j0) {  // lines [j0, lines) one by one
    for (int64_t j = j0; j < c.lines; j++) {
      uint8_t *dj = dev + j * dpitch, *hj = host + j * hpitch;
      hipError_t e = dir == 0 ? hipMemcpyAsync(hj, dj, width, hipMemcpyDeviceToHost, s)
                              : hipMemcpyAsync(dj, hj, width, hipMemcpyHostToDevice, s);
      ++*calls;
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  const int64_t region = copy_region_lines(g, c, lc);
  if (region < 2) return lines_1d(0);
  hipError_t e = dir == 0 ? hipMemcpy2DAsync(host, hpitch, dev, dpitch, width, (size_t)region,
                                             hipMemcpyDeviceToHost, s)
                          : hipMemcpy2DAsync(dev, dpitch, host, hpitch, width, (size_t)region,
                                             hipMemcpyHostToDevice, s);
  if (e == hipErrorInvalidValue || e == hipErrorInvalidPitchValue) {
    (void)hipGetLastError();  // a shape the 2-D path refuses: one copy per line instead
    return lines_1d(0);
  }
  ++*calls;
  if (e != hipSuccess) return e;
  return lines_1d(region);  // the line the region could not hold, if any
}

}  // namespace
}  // namespace kvt

// ---- transfers ----------------------------------------------------------------

// Records one landed event for layers [la, lb) after the work enqueued so far
// on s, and points those layers at it. The event is one that no layer names
// and whose previous recording has completed, taken round-robin from the
// pool's set (the oldest recording comes first); when every free one is still
// in flight, the call waits for the oldest (adding the wait to *blocked_us).
// Caller holds the load direction's lock.
static hipError_t mark_landed(kv_pool *p, int32_t la, int32_t lb, hipStream_t s,
                              double *blocked_us) {
  const size_t E = p->layer_ev.size();
  size_t pick = E, oldest = E;
  for (size_t k = 0; k < E && pick == E; k++) {
    const size_t x = (p->ev_next + k) % E;
    if (p->ev_refs[x] != 0) continue;
    if (!p->ev_recorded[x]) {
      pick = x;
      break;
    }
    const hipError_t q = hipEventQuery(p->layer_ev[x]);
    if (q == hipSuccess) {
      pick = x;
    } else if (q == hipErrorNotReady) {
      if (oldest == E) oldest = x;
    } else {
      return q;
    }
  }
  if (pick == E) {  // 2L + 16 events, at most L named: oldest is set
    const double t0 = now_us();
    const hipError_t w = hipEventSynchronize(p->layer_ev[oldest]);
    *blocked_us += now_us() - t0;
    if (w != hipSuccess) return w;
    pick = oldest;
  }
  const hipError_t e = hipEventRecord(p->layer_ev[pick], s);
  if (e != hipSuccess) return e;
  p->ev_recorded[pick] = 1;
  p->ev_next = (pick + 1) % E;
  for (int32_t l = la; l < lb; l++) {
    const int32_t old = p->layer_src[l].exchange((int32_t)pick);
    if (old >= 0) p->ev_refs[old]--;
    p->ev_refs[pick]++;
  }
  return hipSuccess;
}

// A stream with a hardware queue of its own. HIP maps streams onto a few
// hardware queues round-robin, so a plain stream can land on another stream's
// queue and serialise work that should overlap; a stream created with a CU mask
// gets a hardware queue of its own. The mask enables every compute unit, so it
// does not restrict where kernels run. Default priority.
static hipError_t create_aux_stream(hipStream_t *out) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && cus > 0) {
    std::vector<uint32_t> mask((size_t)(cus + 31) / 32, 0xffffffffu);
    if (cus % 32) mask.back() = (1u << (cus % 32)) - 1u;
    e = hipExtStreamCreateWithCUMask(out, (uint32_t)mask.size(), mask.data());
    if (e == hipSuccess) return e;
    (void)hipGetLastError();
  }
  return hipStreamCreateWithFlags(out, hipStreamNonBlocking);
}

// The staged path's auxiliary streams, one per direction, shared by every pool
// on a device, made on the device's first staged transfer and kept for the
// life of the process: two hardware queues per device however many pools exist
// (more queues than the hardware runs at once would be time-sliced), none for a
// process that never takes the staged path.
struct DeviceStreams {
  hipStream_t aux[2] = {nullptr, nullptr};
};

static hipError_t device_streams(int device, DeviceStreams **out) {
  static std::mutex mu;
  static std::vector<DeviceStreams *> table;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)table.size() <= device) table.resize(device + 1, nullptr);
  if (!table[device]) {
    DeviceStreams *ds = new DeviceStreams;
    hipError_t e = hipSuccess;
    for (int d = 0; d < 2 && e == hipSuccess; d++) e = create_aux_stream(&ds->aux[d]);
    if (e != hipSuccess) {
      for (int d = 0; d < 2; d++)
        if (ds->aux[d]) (void)hipStreamDestroy(ds->aux[d]);
      delete ds;
      return e;
    }
    table[device] = ds;
  }
  *out = table[device];
  return hipSuccess;
}

// True while the other direction has a transfer in flight on this pool on
// another stream than s (its completion event is recorded and not yet
// reached). Work of the other direction queued on s itself runs before this
// call's, not beside it.
static bool other_direction_busy(kv_pool *p, int dir, hipStream_t s) {
  DirState &o = p->dir[1 - dir];
  if (!o.done_recorded.load() || o.done_stream.load() == s) return false;
  return hipEventQuery(o.done) == hipErrorNotReady;
}

// Workgroup cap of a transfer kernel launch (0 = none): the smallest of the
// caps that apply. A direct kernel (kernel and LDS paths) takes the
// direction's own cap, the overlap cap for a load flagged KV_F_LOAD_OVERLAP
// and the duplex cap while the other direction is busy; the staged path's
// device-side passes (HBM to HBM, no host traffic) take only the overlap cap.
static uint32_t kernel_cap(const kv_calib_t &c, int dir, bool overlap, bool duplex,
                           bool direct) {
  uint32_t cap = direct ? (uint32_t)c.kernel_max_workgroups[dir] : 0u;
  auto tighten = [&cap](double limit) {
    if (limit > 0 && (cap == 0 || cap > (uint32_t)limit)) cap = (uint32_t)limit;
  };
  if (overlap) tighten(c.overlap_kernel_max_workgroups);
  if (duplex && direct) tighten(c.duplex_kernel_max_workgroups[dir]);
  return cap;
}

// Dynamic LDS a direct kernel launch asks for per workgroup: a compute unit's
// whole LDS when the launch runs under a grid cap and the direction's
// kernel_cu_exclusive is set, so that its few workgroups each hold a compute
// unit of their own; else none. A workgroup of a capped grid keeps host
// accesses in flight for microseconds, and another kernel's waves on the same
// compute unit then issue their own memory accesses more slowly.
static size_t exclusive_lds(const kv_pool *p, const kv_calib_t &c, int dir, uint32_t cap) {
  return cap != 0 && c.kernel_cu_exclusive[dir] > 0 ? (size_t)p->lds_max : 0;
}

// Wall-clock ticks each of `grid` workgroups spends at least per block (of
// block_bytes) of a direct launch over `blocks` blocks, so that the grid moves
// at most `gbps` GB/s in all (0: unpaced). A grid of one workgroup per block
// has nothing to pace and runs unpaced.
static uint32_t pace_ticks(double block_bytes, uint32_t blocks, uint32_t grid, double gbps,
                           int wall_khz) {
  if (!(gbps > 0) || grid == 0 || grid >= blocks || wall_khz <= 0) return 0;
  const double ticks = std::ceil(block_bytes * grid * wall_khz / (gbps * 1e6));
  return (uint32_t)std::min(std::max(ticks, 1.0), 4294967295.0);
}

// Staged path: makes the direction's staging buffer ready for a call on s that
// moves at most unit_bytes per layer group: the call fills halves of
// min(staged_chunk_bytes, unit_bytes) rounded down to whole rows (stage_use);
// grows the buffer to that (after its previous use has finished) if smaller,
// and orders s after its previous use on another stream.
static int stage_begin(DirState &d, const Geom &g, int64_t unit_bytes, const kv_calib_t &c,
                       hipStream_t s) {
  int64_t want = (int64_t)std::min<double>(c.staged_chunk_bytes, (double)unit_bytes);
  want = std::max<int64_t>(g.R, want / g.R * g.R);
  if (d.stage_cap < want) {
    if (d.stage_pending) {
      hipError_t e = hipEventSynchronize(d.stage_ev);
      d.stage_pending = false;
      if (e != hipSuccess) return hip_fail(e, "waiting for the staging buffer");
    }
    if (d.stage) (void)hipFree(d.stage);
    d.stage = nullptr;
    d.stage_cap = 0;
    if (hipMalloc((void **)&d.stage, 2 * (size_t)want) != hipSuccess) {
      d.stage = nullptr;
      (void)hipGetLastError();
      return fail(KV_ENOMEM, "hipMalloc of the staging buffer failed");
    }
    d.stage_cap = want;
  } else if (d.stage_pending && d.stage_stream != s) {
    hipError_t e = hipStreamWaitEvent(s, d.stage_ev, 0);
    if (e != hipSuccess) return hip_fail(e, "ordering after the staging buffer's last use");
  }
  d.stage_use = want;
  // the halves are free once s reaches this point (the previous call's last
  // use of them is ordered before it)
  d.free_recorded[0] = d.free_recorded[1] = false;
  d.last_half = -1;
  return KV_OK;
}

// Staged path, one layer group [la, lb): the walk rows go through the staging
// halves in chunks (chunk_plan), consecutive chunks (also across groups and
// calls) in alternate halves, so the kernel of one chunk overlaps the copies
// of the other.
//   D2H: aux gathers chunk k (device rows -> half, HBM to HBM) once the half is
//        free; the caller's stream s copies it out, one copy-engine call per
//        host extent piece, then frees the half.
//   H2D: s copies chunk k in once the half is free; aux scatters it to the
//        device rows, then frees the half; the group's landed event is recorded
//        on aux after its last scatter, and the call makes s wait for aux
//        after the last group.
// b is planned for the group; ramp_first / ramp_last select chunk_plan's ramps.
static hipError_t staged_unit(kv_pool *p, DirState &d, int dir, XferArgs b,
                              const int64_t *host_idx, int32_t la, int32_t lb, bool ramp_first,
                              bool ramp_last, uint32_t cap, hipStream_t s, double *blocked_us) {
  const Geom &g = p->g;
  build_extents(g, host_idx, (int64_t)b.n, d.host_run_start, la, lb, &d.extents);
  plan_rows(&b, g.layout, g.ps);
  const int64_t walk_rows = b.total_rows;
  chunk_plan(walk_rows, d.stage_use / g.R, ramp_first, ramp_last, &d.chunk_len);
  size_t x = 0;  // next extent that reaches into the current chunk
  hipError_t e = hipSuccess;
  if (dir == 0) {  // aux starts after everything already queued on s (the KV it reads)
    e = hipEventRecord(d.ev_start, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(d.aux, d.ev_start, 0);
  }
  int last = -1;
  int64_t r0 = 0;
  for (size_t k = 0; k < d.chunk_len.size() && e == hipSuccess; r0 += d.chunk_len[k++]) {
    const int64_t r1 = r0 + d.chunk_len[k];
    const int half = (int)(d.next_half++ & 1);
    last = half;
    uint8_t *buf = d.stage + half * d.stage_cap;
    b.host = buf;
    set_row_range(&b, (uint32_t)r0, (uint32_t)r1);
    hipStream_t kern_s = d.aux;
    uint32_t launched = 0, grid = 0;
    if (dir == 0) {
      if (d.free_recorded[half]) e = hipStreamWaitEvent(kern_s, d.ev_free[half], 0);
      if (e == hipSuccess) {
        e = launch_stage(b, cap, true, kern_s, &launched, &grid);
        d.launches += launched;
        d.last_workgroups = grid;
      }
      if (e == hipSuccess) e = hipEventRecord(d.ev_ready[half], kern_s);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, d.ev_ready[half], 0);
    } else if (d.free_recorded[half]) {
      e = hipStreamWaitEvent(s, d.ev_free[half], 0);
    }
    while (e == hipSuccess && x < d.extents.size() && d.extents[x].walk0 < r1) {
      const Extent &ex = d.extents[x];
      const int64_t a0 = std::max(ex.walk0, r0);
      const int64_t a1 = std::min(ex.walk0 + ex.rows, r1);
      uint8_t *host = p->host + (ex.host0 + (a0 - ex.walk0)) * g.R;
      uint8_t *stage = buf + (a0 - r0) * g.R;
      const size_t nbytes = (size_t)((a1 - a0) * g.R);
      e = dir == 0 ? hipMemcpyAsync(host, stage, nbytes, hipMemcpyDeviceToHost, s)
                   : hipMemcpyAsync(stage, host, nbytes, hipMemcpyHostToDevice, s);
      d.dma++;
      if (ex.walk0 + ex.rows > r1) break;  // continues in the next chunk
      x++;
    }
    if (e != hipSuccess) break;
    if (dir == 0) {
      e = hipEventRecord(d.ev_free[half], s);
    } else {
      e = hipEventRecord(d.ev_ready[half], s);
      if (e == hipSuccess) e = hipStreamWaitEvent(kern_s, d.ev_ready[half], 0);
      if (e == hipSuccess) {
        e = launch_stage(b, cap, false, kern_s, &launched, &grid);
        d.launches += launched;
        d.last_workgroups = grid;
      }
      if (e == hipSuccess) e = hipEventRecord(d.ev_free[half], kern_s);
    }
    d.free_recorded[half] = true;
  }
  if (e == hipSuccess && dir == 1)  // after its last scatter
    e = mark_landed(p, la, lb, d.aux, blocked_us);
  d.last_half = last;
  return e;
}

// Backup on a pool that shares the group writer's host pool: the writer has
// moved (or is moving) the bytes; this call only orders `s` after the writer's
// most recent backup, so the rank's completion is gated by the write, and with
// KV_F_SHARE_CHECK confirms the request names the writer's host rows.
static int shared_backup(kv_pool *p, DirState &d, const int64_t *host_idx, int64_t n,
                         int32_t l0, int32_t l1, hipStream_t s, double t0) {
  HostShare &sh = *p->share;
  hipError_t e = hipSuccess;
  {
    std::lock_guard<std::mutex> sl(sh.mu);
    if (sh.check && (!sh.recorded || request_digest(host_idx, n, l0, l1) != sh.digest))
      return fail(KV_EINVAL,
                  "backup names other host slots or layers than the group writer's latest "
                  "backup (host allocation differs across the group)");
    if (sh.recorded) e = hipStreamWaitEvent(s, sh.written, 0);
  }
  if (e != hipSuccess) return hip_fail(e, "waiting for the group writer's backup");
  e = hipEventRecord(d.done, s);
  if (e != hipSuccess) return hip_fail(e, "recording the completion event");
  d.done_pending = true;
  d.done_stream.store(s);
  d.done_recorded.store(true);
  d.last_path.store(KV_PATH_SHARED);
  d.calls++;
  d.submit_us += now_us() - t0;
  return KV_OK;
}

// Layers per load group: loads go out in groups of `group` layers, each
// followed by one event: one layer per group when a layer alone holds
// load_split_min_bytes, else as many layers as reach it. Backups go out in one
// group.
static int32_t load_group(const Geom &g, const kv_calib_t &c, int dir, int64_t n, int32_t l0,
                          int32_t l1) {
  const int64_t layer_bytes = n * g.C * g.R;
  if (dir != 1 || layer_bytes <= 0) return l1 - l0;
  const double want = c.load_split_min_bytes / (double)layer_bytes;
  return want <= 1.0 ? 1 : (want >= (double)(l1 - l0) ? l1 - l0 : (int32_t)std::ceil(want));
}

// The path selector (AUTO): the modelled time of a validated, non-empty
// request on the kernel, copy-engine and staged paths (times[0..2], us), and
// the path it takes. group: layers per load group (load_group); overlap: a
// load flagged KV_F_LOAD_OVERLAP; duplex: the other direction is busy; cap:
// the kernel paths' grid cap (kernel_cap). Leaves the request's runs, copies,
// host runs and (where listed) staging extents in the vectors.
static int32_t model_path(const Geom &g, const kv_calib_t &c, int dir, const int64_t *dev_idx,
                          const int64_t *host_idx, int64_t n, int32_t l0, int32_t l1,
                          int32_t group, bool overlap, bool duplex, uint32_t cap,
                          std::vector<Run> *runs, std::vector<Copy> *copies,
                          std::vector<int64_t> *run_start, std::vector<Extent> *extents_out,
                          double times[3]) {
  const int64_t nlc_all = (int64_t)(l1 - l0) * g.C;
  const int64_t bytes = n * nlc_all * g.R;
  const int32_t ngroups = (l1 - l0 + group - 1) / group;
  build_runs(g, dev_idx, host_idx, n, runs);
  build_copies(g, *runs, dev_idx, host_idx, copies);
  host_runs(g, host_idx, n, run_start);
  // Exact staging extents cost O(pairs x host runs) to list; past
  // kExtentPlanLimit the upper bound pairs x runs prices the staged path (at
  // one copy per extent it cannot win there anyway).
  const double runs_x_pairs = (double)(run_start->size() - 1) * (double)nlc_all;
  double extents = runs_x_pairs;
  if (g.layout == KV_PAGE_FIRST || runs_x_pairs <= kExtentPlanLimit) {
    build_extents(g, host_idx, n, *run_start, l0, l1, extents_out);
    extents = (double)extents_out->size();
  }
  const double mb = (double)bytes;
  // a capped grid moves what its workgroups can: blocks of 16 KiB of rows
  // per launch, W = min(cap, blocks)
  const int64_t rows_per_block =
      g.R >= (int64_t)kChunksPerBlock * kChunkBytes ? 1 : (int64_t)kChunksPerBlock * kChunkBytes / g.R;
  const double launch_rows = (double)n * std::min<int32_t>(group, l1 - l0) * g.C;
  const double blocks = std::ceil(launch_rows / (double)rows_per_block);
  const double wgs = cap > 0 ? std::min<double>(cap, blocks) : blocks;
  const double rows_all = (double)n * nlc_all;
  // walk rows whose device row does not follow the previous walk row's: each
  // (layer, component) pair starts a run of consecutive device slots inside
  // each group of G positions of the host-order walk
  const int64_t G = g.layout == KV_LAYER_FIRST ? n : (g.layout == KV_PAGE_FIRST ? 1 : g.ps);
  int64_t dev_runs = 0;
  for (int64_t i = 0; i < n; i++)
    if (i % G == 0 || dev_idx[i] != dev_idx[i - 1] + 1) dev_runs++;
  const double jumps = (double)dev_runs * nlc_all;
  const double t_wg =
      ((rows_all * c.kernel_wg_row_ns[dir] + jumps * c.kernel_wg_jump_ns[dir]) * 1e-3 +
       mb / (c.kernel_wg_gbps[dir] * 1e3)) / std::max(wgs, 1.0);
  double t_move = std::max(mb / (c.kernel_gbps[dir] * 1e3), t_wg);
  if (c.kernel_pace_gbps[dir] > 0 && cap > 0 && blocks > cap) {  // a paced grid: past each
    // workgroup's burst, the bytes move at most at the pace
    const double burst = wgs * c.kernel_pace_burst_blocks[dir] * (double)rows_per_block * g.R;
    t_move = std::max(t_move, std::max(0.0, mb - burst) /
                                  (kPaceYield * c.kernel_pace_gbps[dir] * 1e3));
  }
  if (cap > 0 && blocks > cap)  // a capped grid's slow start, whichever bound holds after it
    t_move += c.kernel_wg_start_us[dir] *
              (c.kernel_wg_start_bytes[dir] > 0 ? std::min(1.0, mb / c.kernel_wg_start_bytes[dir])
                                                : 1.0);
  double t_kernel = c.kernel_launch_us[dir] +
                    (ngroups - 1) * (c.kernel_group_us[dir] + c.kernel_link_gap_us[dir]) +
                    t_move;
  double t_dma = (double)copies->size() * nlc_all * c.dma_copy_us[dir] +
                 mb / (c.dma_gbps[dir] * 1e3);
  // the staged path moves page-major layouts in one unit (see transfer); its
  // device-side passes overlap the copies except for the smallest ramp
  // chunk's (chunk_plan), and the ramp adds up to two chunks, each one more
  // launch and one more copy where it splits an extent
  const double units = g.layout == KV_LAYER_FIRST ? (double)ngroups : 1.0;
  const double half = std::min(c.staged_chunk_bytes, mb / units);
  const bool ramped = half * kRampMinDiv >= c.staged_chunk_bytes;
  const double ramp = ramped ? 2.0 : 0.0;
  const double chunks = std::ceil(mb / c.staged_chunk_bytes) + units + ramp;
  double t_staged = (extents + ramp) * c.dma_copy_us[dir] + c.kernel_launch_us[dir] +
                    (chunks - 1) * c.kernel_group_us[dir] + mb / (c.dma_gbps[dir] * 1e3) +
                    (ramped ? half / kRampFirst : half) / (c.staged_gather_gbps * 1e3);
  if (overlap) {
    t_kernel *= 1.0 + c.overlap_kernel_penalty;
    t_dma *= 1.0 + c.overlap_dma_penalty;
    t_staged *= 1.0 + c.overlap_dma_penalty;
    // a page-major staged load is one unit: every layer lands at its end,
    // which a layer-wise consumer cannot overlap
    if (g.layout != KV_LAYER_FIRST) t_staged = std::numeric_limits<double>::infinity();
  }
  if (duplex) t_kernel *= 1.0 + c.duplex_kernel_penalty[dir];
  int32_t path = KV_PATH_KERNEL;
  double best = t_kernel;
  if (t_dma < best) {
    best = t_dma;
    path = KV_PATH_DMA;
  }
  // the staged path also takes HBM bandwidth, compute units and a second
  // stream, so it must win by a margin
  if (t_staged < best * (1.0 - c.staged_min_gain)) path = KV_PATH_STAGED;
  times[0] = t_kernel;
  times[1] = t_dma;
  times[2] = t_staged;
  return path;
}

static int transfer(kv_pool *p, int dir, const int64_t *dev_idx, const int64_t *host_idx,
                    int64_t n, int32_t l0, int32_t l1, void *stream) {
  const double t0 = now_us();
  double blocked = 0;
  if (!p) return fail(KV_EINVAL, "pool is null");
  DirState &d = p->dir[dir];
  std::lock_guard<std::mutex> lock(d.mu);
  const Geom &g = p->g;
  std::string why;
  int rc = validate(g, dir, dev_idx, host_idx, n, l0, l1, (p->flags & KV_F_CHECK_UNIQUE) != 0,
                    &d.uniq, &why);
  if (rc) return fail(rc, why);
  if (n == 0 || l0 == l1) return KV_OK;
  const int64_t nlc_all = (int64_t)(l1 - l0) * g.C;
  if (n * nlc_all >= kMaxRowsPerLaunch)
    return fail(KV_EINVAL, "request has >= 2^31 rows; split it into several calls");

  DeviceGuard dg(p->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipStream_t s = (hipStream_t)stream;
  if (dir == 0 && p->reader) return shared_backup(p, d, host_idx, n, l0, l1, s, t0);
  const int64_t bytes = n * nlc_all * g.R;
  kv_calib_t c;
  {
    std::lock_guard<std::mutex> cl(p->calib_mu);
    c = p->calib;
  }
  int32_t group = load_group(g, c, dir, n, l0, l1);
  const bool overlap = dir == 1 && (p->flags & KV_F_LOAD_OVERLAP) != 0;

  const bool duplex = (p->flags & KV_F_DUPLEX) != 0 || other_direction_busy(p, dir, s);
  const uint32_t cap = kernel_cap(c, dir, overlap, duplex, true);          // kernel paths
  const uint32_t pass_cap = kernel_cap(c, dir, overlap, duplex, false);    // staged passes

  // ---- path selection
  int32_t path = p->path[dir].load();
  bool have_copies = false, have_host_runs = false;
  if (path == KV_PATH_AUTO) {
    double times[3];
    path = model_path(g, c, dir, dev_idx, host_idx, n, l0, l1, group, overlap, duplex, cap,
                      &d.runs, &d.copies, &d.host_run_start, &d.extents, times);
    have_copies = have_host_runs = true;
  }
  if (path == KV_PATH_KERNEL_LDS && g.R > kMaxLdsRowBytes) path = KV_PATH_KERNEL;
  // In page_first / page_first_direct a host page holds every layer of its
  // tokens contiguously; a per-layer unit would cut each page into one small
  // extent per layer. The staged path therefore moves those layouts in one
  // unit, and a load's layers all land together at its end.
  if (path == KV_PATH_STAGED && g.layout != KV_LAYER_FIRST) group = l1 - l0;

  hipError_t e = hipSuccess;
  if (path == KV_PATH_DMA) {
    if (!have_copies) {
      build_runs(g, dev_idx, host_idx, n, &d.runs);
      build_copies(g, d.runs, dev_idx, host_idx, &d.copies);
    }
    for (int32_t la = l0; la < l1 && e == hipSuccess; la += group) {
      const int32_t lb = std::min(l1, la + group);
      for (int32_t l = la; l < lb && e == hipSuccess; l++)
        for (int32_t comp = 0; comp < g.C && e == hipSuccess; comp++)
          for (const Copy &cp : d.copies) {
            e = issue_copy(p, dir, l * g.C + comp, cp, s, &d.dma);
            if (e != hipSuccess) break;
          }
      if (e == hipSuccess && dir == 1) e = mark_landed(p, la, lb, s, &blocked);
    }
    if (e != hipSuccess) return hip_fail(e, "enqueueing copy-engine transfers");
  } else {
    Staging *st = nullptr;
    rc = acquire_staging(d, n, &st, &blocked);
    if (rc) return rc;
    // When a step fails after others of this call were enqueued, the index slot
    // (and, on the staged path, the staging halves) stay in use until the
    // stream passes that work: record that point before reporting the error,
    // so that a later call does not overwrite them under work in flight.
    auto settle = [&](int code) {
      if (path == KV_PATH_STAGED && d.aux && hipEventRecord(d.ev_start, d.aux) == hipSuccess)
        (void)hipStreamWaitEvent(s, d.ev_start, 0);  // s after the call's work on aux
      if (hipEventRecord(st->ev, s) == hipSuccess) st->pending = true;
      if (path == KV_PATH_STAGED && hipEventRecord(d.stage_ev, s) == hipSuccess) {
        d.stage_pending = true;
        d.stage_stream = s;
      }
      return code;
    };
    int64_t *tok = st->pinned;
    for (int64_t i = 0; i < n; i++) {
      tok[2 * i] = dev_idx[i];
      tok[2 * i + 1] = host_key(g, host_idx[i]);
    }
    // Small index arrays are read by the kernels from the mapped pinned buffer
    // (no copy-engine round trip before the first launch); larger ones are
    // copied to the device first, so that the kernels' index reads stay off
    // the host link.
    const bool index_zero_copy = (double)n * 16 <= c.index_zero_copy_max_bytes[dir];
    if (!index_zero_copy) {
      e = hipMemcpyAsync(st->dev, st->pinned, (size_t)n * 16, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return settle(hip_fail(e, "staging indices"));
    }

    XferArgs a{};
    a.tok = index_zero_copy ? st->pinned_dev : st->dev;
    a.dev_tab = p->dev_tab;
    a.host = p->host_dev;
    a.R = g.R;
    a.lc_stride = g.lc_stride;
    a.n = (uint32_t)n;
    if (path == KV_PATH_STAGED) {
      if (!d.aux) {  // the device's auxiliary streams, made on the first staged call
        DeviceStreams *ds = nullptr;
        e = device_streams(p->device, &ds);
        if (e != hipSuccess) return settle(hip_fail(e, "creating the staged path's streams"));
        d.aux = ds->aux[dir];
      }
      rc = stage_begin(d, g, n * (int64_t)std::min<int32_t>(group, l1 - l0) * g.C * g.R, c, s);
      if (rc) return settle(rc);
      if (!have_host_runs) host_runs(g, host_idx, n, &d.host_run_start);
    }
    for (int32_t la = l0; la < l1 && e == hipSuccess; la += group) {
      const int32_t lb = std::min(l1, la + group);
      XferArgs b = a;
      b.lc0 = (uint32_t)(la * g.C);
      b.nlc = (uint32_t)((lb - la) * g.C);
      if (path == KV_PATH_STAGED) {
        const bool ramp = (double)d.stage_use * kRampMinDiv >= c.staged_chunk_bytes;
        e = staged_unit(p, d, dir, b, host_idx, la, lb, ramp && dir == 0,
                        ramp && dir == 1 && lb == l1, pass_cap, s, &blocked);
        continue;  // staged_unit records the group's landed event itself
      } else if (path == KV_PATH_KERNEL_LDS) {
        plan_rows(&b, g.layout, g.ps);  // fills cpr / total_rows
        TileArgs t{};
        b.nblocks = plan_tiles(b, g.layout, &t);
        d.launches++;
        d.last_workgroups = grid_for(b.nblocks, cap);
        b.pace_ticks = pace_ticks((double)t.tile_t * t.tile_lc * g.R, b.nblocks,
                                  (uint32_t)d.last_workgroups,
                                  c.kernel_pace_gbps[dir], p->wall_khz);
        b.pace_burst = (uint32_t)c.kernel_pace_burst_blocks[dir];
        e = launch_tiles_lds(b, t, (uint32_t)d.last_workgroups, dir == 0, s);
      } else {
        const uint32_t blocks = plan_rows(&b, g.layout, g.ps);
        d.launches++;
        d.last_workgroups = grid_for(blocks, cap);
        b.pace_ticks = pace_ticks((double)b.rows_per_block * g.R, blocks,
                                  (uint32_t)d.last_workgroups, c.kernel_pace_gbps[dir],
                                  p->wall_khz);
        b.pace_burst = (uint32_t)c.kernel_pace_burst_blocks[dir];
        e = launch_rows(b, (uint32_t)d.last_workgroups, dir == 0, exclusive_lds(p, c, dir, cap),
                        (int)c.kernel_lane_depth[dir], s);
      }
      if (e == hipSuccess && dir == 1) e = mark_landed(p, la, lb, s, &blocked);
    }
    if (e == hipSuccess && path == KV_PATH_STAGED && dir == 1 && d.last_half >= 0)
      e = hipStreamWaitEvent(s, d.ev_free[d.last_half], 0);  // s ends after aux's last scatter
    if (e != hipSuccess) return settle(hip_fail(e, "enqueueing the transfer"));
    if (path == KV_PATH_STAGED) {
      e = hipEventRecord(d.stage_ev, s);
      if (e != hipSuccess) return settle(hip_fail(e, "recording the staging-buffer event"));
      d.stage_pending = true;
      d.stage_stream = s;
    }
    e = hipEventRecord(st->ev, s);
    if (e != hipSuccess) return settle(hip_fail(e, "recording the staging event"));
    st->pending = true;
  }
  e = hipEventRecord(d.done, s);
  if (e != hipSuccess) return hip_fail(e, "recording the completion event");
  d.done_pending = true;
  d.done_stream.store(s);
  d.done_recorded.store(true);
  if (dir == 0) {  // the writer of the host pool: sharing pools' backups wait for this
    HostShare &sh = *p->share;
    std::lock_guard<std::mutex> sl(sh.mu);
    e = hipEventRecord(sh.written, s);
    if (e != hipSuccess) return hip_fail(e, "recording the host pool's write event");
    sh.recorded = true;
    if (sh.check) sh.digest = request_digest(host_idx, n, l0, l1);
  }
  d.last_path.store(path);
  d.calls++;
  d.bytes += bytes;
  d.blocked_us += blocked;
  d.submit_us += now_us() - t0 - blocked;
  return KV_OK;
}

// ---- the entry point that allocates nothing (kv_transfer_noalloc) -----------

// A kv_transfer_noalloc call's request lives in a file-scope device array:
// positions [0, n) of its raw device slots, of its raw host slots, and its
// index pairs {device slot, host key} (16 bytes each): 8 MiB, 262,144 positions
// at most. Each GPU holds its own copy until the process ends.
constexpr int64_t kNoAllocMaxPositions = int64_t(1) << 18;
static __device__ __align__(256) int64_t scratch[4 * kNoAllocMaxPositions];

// The array's device address on each device, looked up once per device with
// that device current (each GPU holds the array at its own address). Host code
// uses these addresses, never the array's name, for kernel arguments and copies.
constexpr int kNoAllocMaxDevices = 64;
static std::mutex g_scratch_mu;
static int64_t *g_scratch_ptr[kNoAllocMaxDevices] = {};

static int scratch_of(int device, int64_t **out) {
  if (device < 0 || device >= kNoAllocMaxDevices)
    return fail(KV_EINVAL, "device ordinal beyond the no-allocation scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the no-allocation scratch");
    if (!ptr) return fail(KV_EHIP, "hipGetSymbolAddress gave no address for the scratch");
    g_scratch_ptr[device] = static_cast<int64_t *>(ptr);
  }
  *out = g_scratch_ptr[device];
  return KV_OK;
}

// kv_backup (dir 0) / kv_load (dir 1) on the zero-copy kernel path, with the
// request's index arrays copied straight from the caller's arrays into the
// scratch array and paired on the device (pack_pairs), instead of through the
// pool's pinned and device index staging: nothing is allocated on success.
static int transfer_noalloc(kv_pool *p, int dir, const int64_t *dev_idx, const int64_t *host_idx,
                            int64_t n, int32_t l0, int32_t l1, void *stream) {
  const double t0 = now_us();
  double blocked = 0;
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (dir != 0 && dir != 1) return fail(KV_EINVAL, "direction must be 0 (backup) or 1 (load)");
  DirState &d = p->dir[dir];
  std::lock_guard<std::mutex> lock(d.mu);
  const Geom &g = p->g;
  std::string why;
  int rc = validate(g, dir, dev_idx, host_idx, n, l0, l1, (p->flags & KV_F_CHECK_UNIQUE) != 0,
                    &d.uniq, &why, false);
  if (rc) return fail(rc, why);
  if (n > kNoAllocMaxPositions)
    return fail(KV_EINVAL, "n = " + std::to_string(n) +
                               " exceeds the no-allocation call's maximum of 262144 positions");
  if (n == 0 || l0 == l1) return KV_OK;
  const int64_t nlc_all = (int64_t)(l1 - l0) * g.C;
  if (n * nlc_all >= kMaxRowsPerLaunch)
    return fail(KV_EINVAL, "request has >= 2^31 rows; split it into several calls");
  DeviceGuard dg(p->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipStream_t s = (hipStream_t)stream;
  if (dir == 0 && p->reader) return shared_backup(p, d, host_idx, n, l0, l1, s, t0);
  int64_t *sc = nullptr;
  rc = scratch_of(p->device, &sc);
  if (rc) return rc;
  int64_t *raw_dev = sc, *raw_host = sc + kNoAllocMaxPositions, *tok = sc + 2 * kNoAllocMaxPositions;
  kv_calib_t c;
  {
    std::lock_guard<std::mutex> cl(p->calib_mu);
    c = p->calib;
  }
  const int32_t group = load_group(g, c, dir, n, l0, l1);
  const bool overlap = dir == 1 && (p->flags & KV_F_LOAD_OVERLAP) != 0;
  const bool duplex = (p->flags & KV_F_DUPLEX) != 0 || other_direction_busy(p, dir, s);
  const uint32_t cap = kernel_cap(c, dir, overlap, duplex, true);
  hipError_t e = hipMemcpyAsync(raw_dev, dev_idx, (size_t)n * 8, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(raw_host, host_idx, (size_t)n * 8, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = launch_pack_pairs(raw_dev, raw_host, tok, (uint32_t)n, g.layout, (int64_t)g.L * g.C, g.ps,
                          s);
  XferArgs a{};
  a.tok = tok;
  a.dev_tab = p->dev_tab;
  a.host = p->host_dev;
  a.R = g.R;
  a.lc_stride = g.lc_stride;
  a.n = (uint32_t)n;
  for (int32_t la = l0; la < l1 && e == hipSuccess; la += group) {
    const int32_t lb = std::min(l1, la + group);
    XferArgs b = a;
    b.lc0 = (uint32_t)(la * g.C);
    b.nlc = (uint32_t)((lb - la) * g.C);
    const uint32_t blocks = plan_rows(&b, g.layout, g.ps);
    d.launches++;
    d.last_workgroups = grid_for(blocks, cap);
    b.pace_ticks = pace_ticks((double)b.rows_per_block * g.R, blocks,
                              (uint32_t)d.last_workgroups, c.kernel_pace_gbps[dir], p->wall_khz);
    b.pace_burst = (uint32_t)c.kernel_pace_burst_blocks[dir];
    e = launch_rows(b, (uint32_t)d.last_workgroups, dir == 0, exclusive_lds(p, c, dir, cap),
                    (int)c.kernel_lane_depth[dir], s);
    if (e == hipSuccess && dir == 1) e = mark_landed(p, la, lb, s, &blocked);
  }
  if (e != hipSuccess) return hip_fail(e, "enqueueing the no-allocation transfer");
  e = hipEventRecord(d.done, s);
  if (e != hipSuccess) return hip_fail(e, "recording the completion event");
  d.done_pending = true;
  d.done_stream.store(s);
  d.done_recorded.store(true);
  if (dir == 0) {  // the writer of the host pool: sharing pools' backups wait for this
    HostShare &sh = *p->share;
    std::lock_guard<std::mutex> sl(sh.mu);
    e = hipEventRecord(sh.written, s);
    if (e != hipSuccess) return hip_fail(e, "recording the host pool's write event");
    sh.recorded = true;
    if (sh.check) sh.digest = request_digest(host_idx, n, l0, l1);
  }
  d.last_path.store(KV_PATH_KERNEL);
  d.calls++;
  d.bytes += n * nlc_all * g.R;
  d.blocked_us += blocked;
  d.submit_us += now_us() - t0 - blocked;
  return KV_OK;
}

// The staged path's device-side pass on its own (kv_stage): packs (dir 0) or
// unpacks (dir 1) the request's rows between the device buffers and the
// caller's device buffer `stage`, on the caller's stream, in the walk order the
// staged path uses. Uses the direction's index staging.
static int stage_call(kv_pool *p, int dir, const int64_t *dev_idx, int64_t n, int32_t l0,
                      int32_t l1, void *stage, void *stream) {
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (dir != 0 && dir != 1) return fail(KV_EINVAL, "direction must be 0 (pack) or 1 (unpack)");
  DirState &d = p->dir[dir];
  std::lock_guard<std::mutex> lock(d.mu);
  const Geom &g = p->g;
  std::string why;
  int rc = validate_stage(g, dir, dev_idx, n, l0, l1, (p->flags & KV_F_CHECK_UNIQUE) != 0,
                          &d.uniq, &why);
  if (rc) return fail(rc, why);
  if (n == 0 || l0 == l1) return KV_OK;
  const int64_t rows = n * (int64_t)(l1 - l0) * g.C;
  if (rows >= kMaxRowsPerLaunch)
    return fail(KV_EINVAL, "request has >= 2^31 rows; split it into several calls");
  if (!stage || ((uintptr_t)stage & 15u)) return fail(KV_EINVAL, "stage is null or not 16-byte aligned");
  DeviceGuard dg(p->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, stage);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (e == hipSuccess && attr.type == hipMemoryTypeDevice && attr.device == p->device)
    e = hipMemGetAddressRange(&base, &size, stage);
  if (e != hipSuccess || attr.type != hipMemoryTypeDevice || attr.device != p->device ||
      (uint8_t *)stage + rows * g.R > (uint8_t *)base + size) {
    (void)hipGetLastError();
    return fail(KV_EINVAL, "stage is not device memory of the pool's device holding n*layers*C*R "
                           "bytes");
  }
  double blocked = 0;
  Staging *st = nullptr;
  rc = acquire_staging(d, n, &st, &blocked);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  for (int64_t i = 0; i < n; i++) {
    st->pinned[2 * i] = dev_idx[i];
    st->pinned[2 * i + 1] = 0;  // the pass reads device slots only
  }
  e = hipMemcpyAsync(st->dev, st->pinned, (size_t)n * 16, hipMemcpyHostToDevice, s);
  XferArgs a{};
  a.tok = st->dev;
  a.dev_tab = p->dev_tab;
  a.host = (uint8_t *)stage;
  a.R = g.R;
  a.lc_stride = g.lc_stride;
  a.n = (uint32_t)n;
  a.lc0 = (uint32_t)(l0 * g.C);
  a.nlc = (uint32_t)((l1 - l0) * g.C);
  plan_rows(&a, g.layout, g.ps);
  uint32_t launched = 0, grid = 0;
  if (e == hipSuccess) e = launch_stage(a, 0, dir == 0, s, &launched, &grid);
  d.launches += launched;
  if (launched) d.last_workgroups = grid;
  const hipError_t er = hipEventRecord(st->ev, s);  // the index slot is busy until here
  if (er == hipSuccess) st->pending = true;
  if (e != hipSuccess) return hip_fail(e, "enqueueing the staging pass");
  if (er != hipSuccess) return hip_fail(er, "recording the staging event");
  return KV_OK;
}

// kv_calibrate_write_pace: the pool's D2H link rate from timed copy-engine
// copies of its first device buffer into its host pool, and the write-back
// pace set to `fraction` of it. The pool's transfers wait for the measurement
// (both directions' locks, their work in flight drained first).
constexpr int64_t kPaceProbeBytes = int64_t(256) << 20;
constexpr int64_t kPaceProbeMinBytes = int64_t(16) << 20;
constexpr int kPaceProbeCopies = 5;

static int calibrate_write_pace(kv_pool *p, double fraction, void *stream, double *gbps_out) {
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (!(fraction > 0 && fraction <= 1)) return fail(KV_EINVAL, "fraction must be in (0, 1]");
  if (p->reader)
    return fail(KV_EINVAL, "a pool sharing another pool's host pool cannot write into it to "
                           "measure the link; calibrate the group's writer");
  const int64_t buf_bytes = p->g.S_dev * p->g.R;
  const int64_t bytes = std::min({kPaceProbeBytes, p->host_bytes, buf_bytes}) & ~int64_t(4095);
  if (bytes < kPaceProbeMinBytes)
    return fail(KV_EINVAL, "the pool's host pool and first device buffer must each hold 16 MiB "
                           "to measure the link");
  std::lock_guard<std::mutex> l0(p->dir[0].mu);
  std::lock_guard<std::mutex> l1(p->dir[1].mu);
  DeviceGuard dg(p->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipError_t e = drain_direction(p->dir[0]);
  if (e == hipSuccess) e = drain_direction(p->dir[1]);
  if (e != hipSuccess) return hip_fail(e, "pending transfer failed");
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (hipEvent_t &x : ev)
    if (e == hipSuccess) e = hipEventCreate(&x);
  std::vector<double> rates;
  for (int k = 0; k <= kPaceProbeCopies && e == hipSuccess; k++) {  // the first warms up
    e = hipEventRecord(ev[0], s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(p->host, p->bufs[0], (size_t)bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(ev[1], s);
    if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
    float ms = 0;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (e == hipSuccess && k > 0 && ms > 0) rates.push_back((double)bytes / (ms * 1e6));
  }
  for (hipEvent_t x : ev)
    if (x) (void)hipEventDestroy(x);
  if (e != hipSuccess) return hip_fail(e, "timing the link");
  if (rates.empty()) return fail(KV_EHIP, "the link measurement timed no copy");
  std::sort(rates.begin(), rates.end());
  const double gbps = rates[rates.size() / 2];
  if (!(fraction * gbps >= 1))
    return fail(KV_EINVAL, "measured D2H rate " + std::to_string(gbps) +
                               " GB/s gives a pace below 1 GB/s");
  {
    std::lock_guard<std::mutex> cl(p->calib_mu);
    p->calib.kernel_pace_gbps[0] = fraction * gbps;
  }
  if (gbps_out) *gbps_out = gbps;
  return KV_OK;
}

// ---- C ABI ---------------------------------------------------------------------

// Rejects a calibration with a figure out of range (KV_EINVAL).
static int check_calibration(const kv_calib_t *c) {
  for (int d = 0; d < 2; d++)
    if (!(c->kernel_gbps[d] > 0) || !(c->dma_gbps[d] > 0) || !(c->kernel_launch_us[d] >= 0) ||
        !(c->kernel_group_us[d] >= 0) ||
        !(c->dma_copy_us[d] >= 0))
      return fail(KV_EINVAL, "calibration figures must be positive");
  if (!(c->load_split_min_bytes >= 0)) return fail(KV_EINVAL, "load_split_min_bytes must be >= 0");
  for (int d = 0; d < 2; d++)
    if (!(c->kernel_max_workgroups[d] >= 0) || c->kernel_max_workgroups[d] > 4294967295.0)
      return fail(KV_EINVAL, "kernel_max_workgroups must be in [0, 2^32)");
  if (!(c->overlap_kernel_max_workgroups >= 0) || c->overlap_kernel_max_workgroups > 4294967295.0 ||
      !(c->overlap_kernel_penalty >= 0) || !(c->overlap_dma_penalty >= 0))
    return fail(KV_EINVAL, "overlap penalties must be >= 0 and the grid cap in [0, 2^32)");
  if (!(c->index_zero_copy_max_bytes[0] >= 0) || !(c->index_zero_copy_max_bytes[1] >= 0))
    return fail(KV_EINVAL, "index_zero_copy_max_bytes must be >= 0");
  for (int d = 0; d < 2; d++)
    if (!(c->duplex_kernel_max_workgroups[d] >= 0) ||
        c->duplex_kernel_max_workgroups[d] > 4294967295.0)
      return fail(KV_EINVAL, "duplex_kernel_max_workgroups must be in [0, 2^32)");
  for (int d = 0; d < 2; d++)
    if (!(c->kernel_wg_gbps[d] > 0) || !(c->kernel_wg_row_ns[d] >= 0) ||
        !(c->kernel_wg_jump_ns[d] >= 0) ||
        !(c->kernel_wg_start_bytes[d] >= 0) || !(c->kernel_wg_start_us[d] >= 0) ||
        !(c->kernel_link_gap_us[d] >= 0))
      return fail(KV_EINVAL, "kernel_wg_gbps must be > 0, kernel_wg_row_ns, kernel_wg_jump_ns, "
                             "kernel_wg_start_* and kernel_link_gap_us >= 0");
  for (int d = 0; d < 2; d++)
    if (!(c->kernel_pace_gbps[d] == 0 || c->kernel_pace_gbps[d] >= 1) ||
        !(c->kernel_pace_burst_blocks[d] >= 0 && c->kernel_pace_burst_blocks[d] <= 65536) ||
        c->kernel_pace_burst_blocks[d] != std::floor(c->kernel_pace_burst_blocks[d]))
      return fail(KV_EINVAL, "kernel_pace_gbps must be 0 (unpaced) or >= 1, "
                             "kernel_pace_burst_blocks a whole number in [0, 65536]");
  for (int d = 0; d < 2; d++)
    if (c->kernel_cu_exclusive[d] != 0 && c->kernel_cu_exclusive[d] != 1)
      return fail(KV_EINVAL, "kernel_cu_exclusive must be 0 or 1");
  for (int d = 0; d < 2; d++)
    if (c->kernel_lane_depth[d] != 1 && c->kernel_lane_depth[d] != 2 &&
        c->kernel_lane_depth[d] != 4 && c->kernel_lane_depth[d] != 8)
      return fail(KV_EINVAL, "kernel_lane_depth must be 1, 2, 4 or 8");
  if (!(c->duplex_kernel_penalty[0] >= 0) || !(c->duplex_kernel_penalty[1] >= 0) ||
      !(c->staged_chunk_bytes >= 16) ||
      !(c->staged_gather_gbps > 0) || !(c->staged_min_gain >= 0 && c->staged_min_gain < 1))
    return fail(KV_EINVAL, "duplex penalty >= 0, staged chunk >= 16 bytes and gather rate > 0");
  return KV_OK;
}

extern "C" {

const char *kv_last_error(void) { return g_err.c_str(); }

int kv_pool_destroy(kv_pool_t *p) {
  if (!p) return KV_OK;
  int rc = KV_OK;
  {
    DeviceGuard dg(p->device);
    for (DirState &d : p->dir) {
      std::lock_guard<std::mutex> lock(d.mu);
      hipError_t e = drain_direction(d);
      if (e != hipSuccess && rc == KV_OK) rc = hip_fail(e, "pending transfer failed");
      for (Staging &s : d.slots) {
        free_staging(s);
        if (s.ev) (void)hipEventDestroy(s.ev);
      }
      if (d.done) (void)hipEventDestroy(d.done);

      if (d.stage_ev) (void)hipEventDestroy(d.stage_ev);
      if (d.ev_start) (void)hipEventDestroy(d.ev_start);
      for (int h = 0; h < 2; h++) {
        if (d.ev_ready[h]) (void)hipEventDestroy(d.ev_ready[h]);
        if (d.ev_free[h]) (void)hipEventDestroy(d.ev_free[h]);
      }

      if (d.stage) (void)hipFree(d.stage);
    }
    for (hipEvent_t ev : p->layer_ev)
      if (ev) (void)hipEventDestroy(ev);
    if (p->dev_tab) (void)hipFree(p->dev_tab);
  }
  p->share.reset();  // the host pool goes with the group's last pool
  delete p;
  return rc;
}

// kv_pool_create (group == nullptr: allocates the host pool) and
// kv_pool_create_shared (shares group's host pool).
static int create_pool(const kv_pool_desc_t *desc, kv_pool *group, kv_pool_t **out) {
  if (!desc || !out) return fail(KV_EINVAL, "desc and out must be non-null");
  *out = nullptr;
  Geom g;
  std::string why;
  int rc = make_geom(&desc->geom, &g, &why);
  if (rc) return fail(rc, why);
  if (!desc->device_buffers) return fail(KV_EINVAL, "device_buffers is null");
  if (group) {
    const Geom &w = group->g;
    if (g.L != w.L || g.C != w.C || g.R != w.R || g.S_host != w.S_host || g.ps != w.ps ||
        g.layout != w.layout)
      return fail(KV_EINVAL,
                  "a pool sharing a host pool must have the group's geometry (all but device_slots)");
  } else if (desc->numa_node >= 0 && !numa_node_exists(desc->numa_node)) {
    return fail(KV_EINVAL, "numa_node " + std::to_string(desc->numa_node) + " does not exist");
  } else if (desc->numa_node >= 0 && (desc->flags & KV_F_HOST_INTERLEAVE)) {
    return fail(KV_EINVAL, "numa_node and KV_F_HOST_INTERLEAVE are exclusive");
  }
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (desc->device < 0 || desc->device >= ndev)
    return fail(KV_EINVAL, "device " + std::to_string(desc->device) + " does not exist");
  DeviceGuard dg(desc->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");

  const int64_t nbuf = (int64_t)g.L * g.C;
  const int64_t buf_bytes = g.S_dev * g.R;
  kv_pool *p = new kv_pool(g.L);
  p->g = g;
  p->device = desc->device;
  p->flags = desc->flags;
  p->numa = desc->numa_node;
  default_calibration(&p->calib);
  p->bufs.resize(nbuf);
  for (int64_t k = 0; k < nbuf; k++) {
    uint8_t *b = static_cast<uint8_t *>(desc->device_buffers[k]);
    if (!b || ((uintptr_t)b & 15u)) {
      delete p;
      return fail(KV_EINVAL, "device buffer " + std::to_string(k) + " is null or not 16-byte aligned");
    }
    // The buffer must be device memory of this device holding S_dev*R bytes.
    hipPointerAttribute_t attr;
    e = hipPointerGetAttributes(&attr, b);
    if (e != hipSuccess || attr.type != hipMemoryTypeDevice || attr.device != desc->device) {
      (void)hipGetLastError();
      delete p;
      return fail(KV_EINVAL, "device buffer " + std::to_string(k) +
                                 " is not device memory of device " + std::to_string(desc->device));
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, b);
    if (e != hipSuccess || (uint8_t *)b + buf_bytes > (uint8_t *)base + size) {
      (void)hipGetLastError();
      delete p;
      return fail(KV_EINVAL, "device buffer " + std::to_string(k) + " is smaller than S_dev*R bytes");
    }
    p->bufs[k] = b;
  }

  if (desc->flags & KV_F_CHECK_UNIQUE) {  // tables kv_transfer_noalloc checks with
    try {
      p->dir[0].uniq.stamp.assign((size_t)std::min(g.S_host, kStampSlotsPresize), 0u);
      p->dir[1].uniq.stamp.assign((size_t)std::min(g.S_dev, kStampSlotsPresize), 0u);
    } catch (const std::bad_alloc &) {
      delete p;
      return fail(KV_ENOMEM, "allocating the uniqueness tables");
    }
  }
  if (group) {  // the group's host pool
    p->share = group->share;
    p->reader = true;
    p->host = p->share->host;
    p->host_bytes = p->share->bytes;
  } else {
    // host pool: pinned, mapped for the device and portable (a pool on another
    // device may share it), optionally bound to a node
    p->host_bytes = nbuf * g.S_host * g.R;
    unsigned int hflags = hipHostMallocMapped | hipHostMallocPortable |
                          ((desc->flags & KV_F_HOST_NONCOHERENT) ? hipHostMallocNonCoherent
                                                                 : hipHostMallocCoherent);
    int old_mode = 0;
    unsigned long old_mask = 0;
    bool bound = false;
    if (desc->numa_node >= 0) {
      bound = set_thread_policy(kMpolBind, 1ul << desc->numa_node, &old_mode, &old_mask);
      if (!bound) {
        delete p;
        return fail(KV_EINVAL,
                    "set_mempolicy to node " + std::to_string(desc->numa_node) + " failed");
      }
      hflags |= hipHostMallocNumaUser;
    } else if (desc->flags & KV_F_HOST_INTERLEAVE) {
      const unsigned long nodes = online_numa_nodes();
      bound = nodes != 0 && set_thread_policy(kMpolInterleave, nodes, &old_mode, &old_mask);
      if (!bound) {
        delete p;
        return fail(KV_EINVAL, "set_mempolicy to interleave over the online nodes failed");
      }
      hflags |= hipHostMallocNumaUser;
    }
    uint8_t *host = nullptr;
    e = hipHostMalloc((void **)&host, (size_t)p->host_bytes, hflags);
    if (bound) restore_thread_policy(old_mode, old_mask);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      kv_pool_destroy(p);
      return fail(KV_ENOMEM, "hipHostMalloc of " + std::to_string(nbuf * g.S_host * g.R) +
                                 " bytes failed: " + hipGetErrorString(e));
    }
    p->share = std::make_shared<HostShare>();
    p->share->device = desc->device;
    p->share->host = host;
    p->share->bytes = p->host_bytes;
    p->share->check = (desc->flags & KV_F_SHARE_CHECK) != 0;
    p->host = host;
    e = hipEventCreateWithFlags(&p->share->written, hipEventDisableTiming);
    if (e != hipSuccess) {
      kv_pool_destroy(p);
      return hip_fail(e, "creating the host pool's write event");
    }
  }
  void *hd = nullptr;
  e = hipHostGetDevicePointer(&hd, p->host, 0);
  if (e != hipSuccess) {
    kv_pool_destroy(p);
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  p->host_dev = (uint8_t *)hd;
  e = hipDeviceGetAttribute(&p->wall_khz, hipDeviceAttributeWallClockRate, p->device);
  if (e != hipSuccess || p->wall_khz <= 0) {
    kv_pool_destroy(p);
    return e != hipSuccess ? hip_fail(e, "reading the device's wall-clock rate")
                           : fail(KV_EHIP, "the device reports no wall-clock rate");
  }
  e = hipDeviceGetAttribute(&p->lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, p->device);
  if (e != hipSuccess || p->lds_max < 0) {
    kv_pool_destroy(p);
    return e != hipSuccess ? hip_fail(e, "reading the device's LDS per workgroup")
                           : fail(KV_EHIP, "the device reports a negative LDS size");
  }

  e = hipMalloc((void **)&p->dev_tab, (size_t)nbuf * sizeof(uint8_t *));
  if (e == hipSuccess)
    e = hipMemcpy(p->dev_tab, p->bufs.data(), (size_t)nbuf * sizeof(uint8_t *),
                  hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    kv_pool_destroy(p);
    return hip_fail(e, "device buffer table");
  }
  const size_t nev = 2 * (size_t)g.L + 16;
  p->layer_ev.assign(nev, nullptr);
  p->ev_refs.assign(nev, 0);
  p->ev_recorded.assign(nev, 0);
  for (size_t k = 0; k < nev && e == hipSuccess; k++)
    e = hipEventCreateWithFlags(&p->layer_ev[k], hipEventDisableTiming);
  for (DirState &d : p->dir) {
    if (e == hipSuccess) e = hipEventCreateWithFlags(&d.done, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&d.stage_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&d.ev_start, hipEventDisableTiming);
    for (int h = 0; h < 2; h++) {
      if (e == hipSuccess) e = hipEventCreateWithFlags(&d.ev_ready[h], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&d.ev_free[h], hipEventDisableTiming);
    }

    for (Staging &s : d.slots)
      if (e == hipSuccess) e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    kv_pool_destroy(p);
    return hip_fail(e, "creating events");
  }
  *out = p;
  return KV_OK;
}

int kv_pool_create(const kv_pool_desc_t *desc, kv_pool_t **out) {
  return guarded("kv_pool_create", [&] { return create_pool(desc, nullptr, out); });
}

int kv_pool_create_shared(const kv_pool_desc_t *desc, kv_pool_t *group, kv_pool_t **out) {
  if (out) *out = nullptr;
  if (!group) return fail(KV_EINVAL, "group is null");
  return guarded("kv_pool_create_shared", [&] { return create_pool(desc, group, out); });
}

void *kv_pool_host_ptr(const kv_pool_t *p) { return p ? p->host : nullptr; }
int64_t kv_pool_host_bytes(const kv_pool_t *p) { return p ? p->host_bytes : 0; }

int kv_backup(kv_pool_t *p, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
              int32_t layer_begin, int32_t layer_end, void *stream) {
  return guarded("kv_backup", [&] {
    return transfer(p, 0, dev_idx, host_idx, n, layer_begin, layer_end, stream);
  });
}

int kv_load(kv_pool_t *p, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
            int32_t layer_begin, int32_t layer_end, void *stream) {
  return guarded("kv_load", [&] {
    return transfer(p, 1, dev_idx, host_idx, n, layer_begin, layer_end, stream);
  });
}

int kv_transfer_noalloc(kv_pool_t *p, int32_t direction, const int64_t *dev_idx,
                        const int64_t *host_idx, int64_t n, int32_t layer_begin,
                        int32_t layer_end, void *stream) {
  return guarded("kv_transfer_noalloc", [&] {
    return transfer_noalloc(p, direction, dev_idx, host_idx, n, layer_begin, layer_end, stream);
  });
}

int kv_stage(kv_pool_t *p, int32_t direction, const int64_t *dev_idx, int64_t n,
             int32_t layer_begin, int32_t layer_end, void *stage, void *stream) {
  return guarded("kv_stage", [&] {
    return stage_call(p, direction, dev_idx, n, layer_begin, layer_end, stage, stream);
  });
}

int kv_load_layer(kv_pool_t *p, int32_t layer, void *compute_stream) {
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (layer < 0 || layer >= p->g.L)
    return fail(KV_EINVAL, "layer " + std::to_string(layer) + " is outside [0, L)");
  const int32_t src = p->layer_src[layer].load();
  if (src < 0) return KV_OK;
  DeviceGuard dg(p->device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipError_t e = hipStreamWaitEvent((hipStream_t)compute_stream, p->layer_ev[src], 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  return KV_OK;
}

int kv_stream_create(int32_t device, void **out) {
  if (!out) return fail(KV_EINVAL, "out is null");
  *out = nullptr;
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev)
    return fail(KV_EINVAL, "device " + std::to_string(device) + " does not exist");
  DeviceGuard dg(device);
  if (dg.err != hipSuccess) return hip_fail(dg.err, "hipSetDevice");
  hipStream_t st = nullptr;
  int rc = guarded("kv_stream_create", [&] {
    e = create_aux_stream(&st);
    return KV_OK;
  });
  if (rc) return rc;
  if (e != hipSuccess) return hip_fail(e, "creating a stream");
  *out = st;
  return KV_OK;
}

int kv_stream_destroy(void *stream) {
  if (!stream) return KV_OK;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  hipError_t e2 = hipStreamDestroy((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "synchronising the stream");
  if (e2 != hipSuccess) return hip_fail(e2, "destroying the stream");
  return KV_OK;
}

int kv_set_path(kv_pool_t *p, int32_t path) {
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (path < KV_PATH_AUTO || path > KV_PATH_STAGED) return fail(KV_EINVAL, "unknown path");
  p->path[0].store(path);
  p->path[1].store(path);
  return KV_OK;
}

int kv_set_direction_path(kv_pool_t *p, int32_t direction, int32_t path) {
  if (!p) return fail(KV_EINVAL, "pool is null");
  if (direction != 0 && direction != 1) return fail(KV_EINVAL, "direction must be 0 or 1");
  if (path < KV_PATH_AUTO || path > KV_PATH_STAGED) return fail(KV_EINVAL, "unknown path");
  p->path[direction].store(path);
  return KV_OK;
}

int32_t kv_last_path(const kv_pool_t *p, int32_t direction) {
  if (!p || (direction != 0 && direction != 1)) return -1;
  return p->dir[direction].last_path.load();
}

int kv_set_calibration(kv_pool_t *p, const kv_calib_t *c) {
  if (!p || !c) return fail(KV_EINVAL, "pool and calibration must be non-null");
  const int rc = check_calibration(c);
  if (rc) return rc;
  std::lock_guard<std::mutex> lock(p->calib_mu);
  p->calib = *c;
  return KV_OK;
}

int kv_get_calibration(const kv_pool_t *p, kv_calib_t *c) {
  if (!p || !c) return fail(KV_EINVAL, "pool and calibration must be non-null");
  std::lock_guard<std::mutex> lock(const_cast<kv_pool *>(p)->calib_mu);
  *c = p->calib;
  return KV_OK;
}

int kv_get_stats(const kv_pool_t *p, kv_stats_t *out) {
  if (!p || !out) return fail(KV_EINVAL, "pool and out must be non-null");
  for (int d = 0; d < 2; d++) {
    DirState &s = const_cast<kv_pool *>(p)->dir[d];
    std::lock_guard<std::mutex> lock(s.mu);
    out->calls[d] = s.calls;
    out->bytes[d] = s.bytes;
    out->kernel_launches[d] = s.launches;
    out->dma_copies[d] = s.dma;
    out->submit_us[d] = s.submit_us;
    out->blocked_us[d] = s.blocked_us;
    out->last_workgroups[d] = s.last_workgroups;
  }
  return KV_OK;
}

int kv_calibrate_write_pace(kv_pool_t *p, double fraction, void *stream, double *d2h_gbps) {
  return guarded("kv_calibrate_write_pace",
                 [&] { return calibrate_write_pace(p, fraction, stream, d2h_gbps); });
}

int kv_default_calibration(kv_calib_t *c) {
  if (!c) return fail(KV_EINVAL, "calibration is null");
  default_calibration(c);
  return KV_OK;
}

int32_t kv_model_path(const kv_geometry_t *geom, const kv_calib_t *calib, int32_t direction,
                      const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                      int32_t layer_begin, int32_t layer_end, uint32_t flags,
                      double *times_us) {
  return guarded("kv_model_path", [&]() -> int {
    if (!geom || !calib || !times_us)
      return fail(KV_EINVAL, "geom, calib and times_us must be non-null");
    if (direction != 0 && direction != 1) return fail(KV_EINVAL, "direction must be 0 or 1");
    Geom g;
    std::string why;
    int rc = make_geom(geom, &g, &why);
    if (rc) return fail(rc, why);
    rc = check_calibration(calib);
    if (rc) return rc;
    rc = validate(g, direction, dev_idx, host_idx, n, layer_begin, layer_end, false, nullptr,
                  &why);
    if (rc) return fail(rc, why);
    if (n == 0 || layer_begin == layer_end) return fail(KV_EINVAL, "empty request");
    if (n * (int64_t)(layer_end - layer_begin) * g.C >= kMaxRowsPerLaunch)
      return fail(KV_EINVAL, "request has >= 2^31 rows; split it into several calls");
    const bool overlap = direction == 1 && (flags & KV_F_LOAD_OVERLAP) != 0;
    const bool duplex = (flags & KV_F_DUPLEX) != 0;
    const uint32_t cap = kernel_cap(*calib, direction, overlap, duplex, true);
    const int32_t group = load_group(g, *calib, direction, n, layer_begin, layer_end);
    std::vector<Run> runs;
    std::vector<Copy> copies;
    std::vector<int64_t> run_start;
    std::vector<Extent> extents;
    return (int)model_path(g, *calib, direction, dev_idx, host_idx, n, layer_begin, layer_end,
                           group, overlap, duplex, cap, &runs, &copies, &run_start, &extents,
                           times_us);
  });
}

}  // extern "C"
