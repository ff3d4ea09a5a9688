/*
 * kvtier.h — C ABI of the cross-tier KV transfer library (libkvtier.so).
 *
 * What it moves. A hierarchical prefix cache keeps KV in device HBM ("L1") and
 * spills or restores it through a pinned host DRAM pool ("L2"). Write-back
 * (device -> host, "D2H") and load (host -> device, "H2D") are indexed copies
 * of whole KV rows between the two tiers (pages: "Tuning SGLang HiCache L2 on
 * Kunlunxin P800/P900", sections 1.2 and 2.1; "HiCache system design",
 * section "data transfer optimisation").
 *
 * Vocabulary used below.
 *   L   layers, C components per layer (2 = K and V; 1 = an MLA latent).
 *   R   row bytes: one token's K (or V, or latent) for one layer = H*D*elem.
 *   S_dev  token slots in each device buffer; S_host token slots in the host pool.
 *   ps  page size in tokens.
 *   A "row" is R contiguous bytes. Values are moved as raw bytes, never
 *   interpreted, so any element type (bf16, fp8 with NaN patterns, ...) is fine.
 *
 * Device pool (L1). Layer-first: L*C separate device buffers B[l][c], each
 * S_dev*R bytes, row d at B[l][c] + d*R ("different layers are different
 * buffers": Kunlunxin tuning page, section 2.1; "L1 is fixed layer-first":
 * Baidu KV cache page, section "L2 layout choice"). The buffers are BORROWED:
 * the caller (e.g. torch) owns them and keeps them alive until
 * kv_pool_destroy().
 *
 * Host pool (L2). One byte array of L*C*S_host*R bytes, OWNED by the library,
 * allocated pinned and mapped for the device. Host slot h of layer l,
 * component c lives at row host_row(l,c,h), byte offset host_row*R:
 *   KV_LAYER_FIRST        dims (layer, comp, slot, row):  (l*C + c)*S_host + h
 *   KV_PAGE_FIRST         dims (slot, layer, comp, row):  (h*L + l)*C + c
 *   KV_PAGE_FIRST_DIRECT  dims (page, layer, comp, offset-in-page, row):
 *                         ((h/ps*L + l)*C + c)*ps + h%ps
 * The layer_first and page_first_direct dimension orders are the ones the
 * Kunlunxin tuning page gives in section 2.1 ("(layer, size, 1, kv_dim)" and
 * "(page_num, layer_num, page_size, 1, kv_dim)"); page_first keeps a page
 * contiguous and moves at one-token-per-layer granularity (HiCache system
 * design page, section "data transfer optimisation"). Where the pages are
 * silent we read: the component axis sits directly inside the layer axis in
 * all three layouts, and page_first is token-outer, layer-inner.
 *
 * Asynchrony. kv_backup/kv_load return once the work is ENQUEUED on the given
 * HIP stream; nothing blocks on the transfer ("start_writing()/start_loading()
 * only enqueue; dedicated threads submit on private streams": Kunlunxin tuning
 * page section 2.2; Baidu page "bidirectional async transfer"). Completion is
 * observed through the stream or through kv_load_layer().
 *
 * Threads. One backup thread and one load thread may call concurrently on one
 * pool (each direction has its own internal state and lock). Calls of the same
 * direction from several threads are serialised by that lock.
 *
 * Errors. Every int-returning call returns KV_OK (0) or a negative KV_E* code;
 * kv_last_error() gives a message for the calling thread. When validation
 * fails nothing is enqueued and no byte of either pool is modified. A HIP
 * failure of already-enqueued work surfaces at a later call or at destroy.
 * No C++ exception leaves the library: if the library's own host bookkeeping
 * cannot be allocated, the call returns KV_ENOMEM (a transfer may then have
 * been partly enqueued).
 */
#ifndef KVTIER_H
#define KVTIER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define KV_OK       0
#define KV_EINVAL  (-1) /* bad argument or precondition (null pointer, n<0, bad layer range, R%16, S_host%ps, ...) */
#define KV_ERANGE  (-2) /* an index is outside [0, S_dev) or [0, S_host) */
#define KV_EDUP    (-3) /* a destination slot appears twice in one call (only with KV_F_CHECK_UNIQUE) */
#define KV_ENOMEM  (-4) /* host or device allocation failed */
#define KV_EHIP    (-5) /* a HIP runtime call failed */

/* ---- host layouts ------------------------------------------------------ */
typedef enum {
  KV_LAYER_FIRST = 0,
  KV_PAGE_FIRST = 1,
  KV_PAGE_FIRST_DIRECT = 2
} kv_layout_t;

/* ---- execution paths ---------------------------------------------------
 * KV_PATH_AUTO        per call, pick the cheapest of KERNEL, DMA and STAGED
 *                     from the byte count, the number of DMA copies and of
 *                     staging extents the request needs, using the pool's
 *                     calibration (kv_calib_t).
 * KV_PATH_KERNEL      zero-copy gather/scatter kernel: the GPU reads/writes the
 *                     mapped host pool directly, 8 bytes per lane (a wave's
 *                     access covers 512 consecutive bytes), rows taken in
 *                     host-address order.
 * KV_PATH_KERNEL_LDS  as KERNEL, but each workgroup stages a tile of rows in
 *                     LDS: read in source order, written in destination order
 *                     (the page_first <-> layer_first transpose).
 * KV_PATH_DMA         coalesced copy-engine path: maximal contiguous runs,
 *                     uniform-stride runs merged into 2-D copies, issued as
 *                     hipMemcpyAsync / hipMemcpy2DAsync on the stream.
 * KV_PATH_STAGED      batched gather/scatter through a device staging buffer:
 *                     a kernel gathers the rows into host-address order in
 *                     HBM (or scatters them from it), and the copy engines move
 *                     each contiguous host extent in one call (Baidu KV cache
 *                     page, "DMA segment explosion & batched gather/scatter").
 *                     A page of a page-first layout is one extent, so the link
 *                     moves on the copy engines with few calls whatever the
 *                     device-side fragmentation.                            */
typedef enum {
  KV_PATH_AUTO = 0,
  KV_PATH_KERNEL = 1,
  KV_PATH_KERNEL_LDS = 2,
  KV_PATH_DMA = 3,
  KV_PATH_STAGED = 4,
  KV_PATH_SHARED = 5 /* reported by kv_last_path only: the backup of a pool that
                        shares another pool's host pool (kv_pool_create_shared)
                        moved no data and waited for the writer's backup */
} kv_path_t;

/* ---- pool flags -------------------------------------------------------- */
#define KV_F_CHECK_UNIQUE     0x1u /* reject duplicate destination slots (KV_EDUP) */
#define KV_F_HOST_NONCOHERENT 0x2u /* allocate the host pool non-coherent (coarse-grained) instead of coherent */
#define KV_F_DUPLEX           0x8u /* backups and loads on this pool run at the same time: the
                                      selector charges the kernel path the duplex penalty and
                                      the kernel paths run on the duplex grids
                                      (duplex_kernel_max_workgroups).
                                      Without it both apply only while the other
                                      direction has a transfer in flight at submission on
                                      another stream (work queued on the same stream runs
                                      before this call, not beside it). */
#define KV_F_HOST_INTERLEAVE  0x20u /* spread the host pool's pages across all online NUMA
                                       nodes (interleaved placement: capacity first; Baidu KV
                                       cache page, "shared buffer placement"); exclusive with
                                       numa_node >= 0 (socket-local placement) */
#define KV_F_SHARE_CHECK      0x10u /* on the writer of a shared host pool (kv_pool_create_shared):
                                       each backup of a sharing pool must name the same host
                                       slots and layer range as the writer's latest backup,
                                       else KV_EINVAL (host allocation differs across the group) */
#define KV_F_LOAD_OVERLAP     0x4u /* loads on this pool run while compute kernels occupy the GPU
                                      (layer-wise load during the forward pass): the selector
                                      charges each path the compute time it steals, the
                                      kernel path runs on a capped grid, and in page_first /
                                      page_first_direct AUTO leaves out the staged path (it
                                      lands every layer at the end of the load) */

/* Geometry of one pool. Needs no GPU; the planner calls below take it alone. */
typedef struct {
  int32_t num_layers;     /* L  >= 1 */
  int32_t num_components; /* C  >= 1 (2 = K,V; 1 = MLA latent) */
  int64_t row_bytes;      /* R  >= 16, R % 16 == 0, R <= 2^30 (the kernels count a
                             row's chunks in 32 bits) */
  int64_t device_slots;   /* S_dev >= 1 */
  int64_t host_slots;     /* S_host >= 1, S_host % page_size == 0 */
  int32_t page_size;      /* ps >= 1 */
  int32_t host_layout;    /* kv_layout_t */
} kv_geometry_t;

typedef struct {
  kv_geometry_t geom;
  /* L*C device buffer base pointers, index l*C + c, each S_dev*R bytes and
   * 16-byte aligned. The array itself is copied during kv_pool_create; the
   * buffers it points to are borrowed. */
  void *const *device_buffers;
  int32_t device;    /* HIP device ordinal the buffers live on */
  int32_t numa_node; /* -1: no binding; else the host pool's pages are bound to this node
                        (0..63) */
  uint32_t flags;    /* KV_F_* */
} kv_pool_desc_t;

/* Selector calibration: modelled time of a call on each path.
 *   t_kernel = kernel_launch_us
 *              + (launches - 1) * (kernel_group_us + kernel_link_gap_us)
 *              + bytes / kernel_gbps
 *   t_dma    = copies * dma_copy_us + bytes / dma_gbps
 * kernel_launch_us is the fixed cost of a call's first launch (launch, index
 * staging, ramp), kernel_group_us the gap each further launch of the same
 * call adds, and kernel_link_gap_us the time the host link then also stands
 * idle while one launch drains and the next ramps up (the staged path's
 * launches overlap its copies, so it pays kernel_group_us alone). On a
 * capped grid of W workgroups the kernel is limited by what W workgroups
 * move: bytes / kernel_gbps is replaced by the larger of itself,
 * ((rows * kernel_wg_row_ns + jumps * kernel_wg_jump_ns) * 1e-3
 *  + bytes / (kernel_wg_gbps * 1e3)) / W
 * and, when paced, the pace term under kernel_pace_burst_blocks below, plus
 * kernel_wg_start_us * min(1, bytes / kernel_wg_start_bytes)
 * (microseconds), rows being the call's n * layers * C rows and jumps those
 * rows of the host-order walk whose device row does not follow the previous
 * walk row's (layers * C times the runs of consecutive device slots within
 * the walk's groups of positions: the whole request in layer_first, each
 * position in page_first, each page in page_first_direct): a capped grid
 * moves the first kernel_wg_start_bytes of a call more slowly, which costs up
 * to kernel_wg_start_us more whichever bound holds (a capped grid has W < the
 * launch's blocks).
 * The rates are fitted per direction on the target machine to the time a
 * call takes less its modelled fixed costs.
 * load_split_min_bytes: kv_load goes out in groups of consecutive layers, one
 * kernel launch (or one batch of copies) and one landed event per group; a
 * group is one layer when a layer of the request holds at least this many
 * bytes, else the fewest layers that reach it. Small loads thus pay for few
 * launches and events, large ones signal every layer as soon as it lands.
 * kernel_max_workgroups: cap on the workgroups one direct transfer kernel
 * (kernel and LDS paths) launches (0 = one per block of work; the staged
 * path's device-side passes, HBM to HBM, are not capped by it). The kernels
 * stride over their work, so a cap moves the same bytes while leaving compute
 * units free for kernels on other streams (e.g. the layer that was just
 * loaded). Default: 18 for a backup, none for a load. A write-back kernel on a
 * large grid keeps so many posted host writes queued that HBM-bound kernels
 * running beside it slow by up to ~46x; the slowdown follows the writes in
 * flight, and 18 workgroups of two chunks per lane (kernel_lane_depth), paced,
 * move ~96-98% of the full grid's rate while they slow by ~1.16x (the copy
 * engines: ~1.12-1.15x). Set [0] to 0 for the full grid when nothing else runs
 * during backups.
 * kernel_pace_gbps: on the kernel and LDS paths, > 0 holds a launch's
 * workgroups to this total rate: each starts its blocks of work (tiles on the
 * LDS path) at least grid * block bytes / rate apart on the device's
 * constant-rate wall clock, with one block of catch-up after a stall; each
 * workgroup's first interval is offset by its share of one, so the grid's
 * blocks go out spread over it. Each write-back workgroup issues up to ~3.3
 * GB/s of posted host writes at two chunks per lane (~6.6 at eight); a grid
 * that issues more than the host link drains queues them in the memory system
 * and falls to ~40 GB/s, so the pace must stay under the link's D2H rate.
 * Default: 54 for a backup (~2% under the lowest D2H drain rate measured on
 * an MI355X's PCIe Gen5 x16 link; a caller that measures its own link's D2H
 * copy rate can pace at ~0.98 of it), 0 (unpaced) for a load.
 * kernel_pace_burst_blocks: a paced workgroup's first max(1, this) blocks go
 * out at once and its pacing starts from the last of them: the start of a call
 * is latency-bound, and pacing it from the first block slows small calls.
 * Default: 32 for a backup. On a capped grid of W workgroups the model's
 * kernel time before the slow start is at least (bytes - W * burst blocks *
 * block bytes) / (0.99 * kernel_pace_gbps), a block being the rows of 16 KiB
 * or one row if longer (a paced grid delivered 98-99% of its pace past its
 * start).
 * With KV_F_LOAD_OVERLAP, a load's modelled time on each path is multiplied
 * by (1 + penalty): overlap_kernel_penalty / overlap_dma_penalty are the
 * fractions of the transfer time by which a concurrent HBM-bound kernel is
 * slowed, measured per path; and the kernel path launches at most
 * overlap_kernel_max_workgroups workgroups (default 24, which keep the link
 * full; their workgroups take compute units of their own, kernel_cu_exclusive).
 * duplex_kernel_max_workgroups: cap on the workgroups of a kernel-path
 * transfer while the other direction is busy (KV_F_DUPLEX, or a transfer of
 * the other direction in flight at submission on another stream); [0] for a
 * backup, [1] for a load, 0 = no cap; defaults 8 and 32. A load's kernel holds
 * the link with 32 workgroups; a write-back kernel with a small grid leaves the
 * load most of the link and, together with the load's cap, leaves compute
 * units free for the other direction's kernels. The staged path's device-side
 * passes are not capped by it.
 * The staged path moves a unit (all layers, or one load group in layer_first)
 * through two staging halves of min(staged_chunk_bytes, unit bytes) each, in
 * chunks that fill a half, except where a device-side pass cannot overlap a
 * copy: on a half of at least staged_chunk_bytes / 16, a backup's first chunks
 * and a load's last ones grow by 8x from 1/64 of a half. It is modelled as
 * (extents + ramp) * dma_copy_us + kernel_launch_us + (chunks - 1) *
 * kernel_group_us + bytes / dma_gbps + first / staged_gather_gbps, with
 * ramp = 2 chunks and first = half / 64 where the ramp applies (else ramp = 0
 * and first = half): the device-side passes overlap the copies except for
 * that one. */
typedef struct {
  double kernel_launch_us[2]; /* [0] = D2H backup, [1] = H2D load */
  double kernel_gbps[2];
  double dma_copy_us[2];
  double dma_gbps[2];
  double load_split_min_bytes;
  double kernel_max_workgroups[2];
  double overlap_kernel_penalty;
  double overlap_dma_penalty;
  double overlap_kernel_max_workgroups;
  double duplex_kernel_penalty[2]; /* kernel-path slowdown of this direction while the other
                                      one is busy ([0] backup beside a load, [1] load beside a
                                      backup) */
  double staged_chunk_bytes;    /* staged path: staging buffer size per direction */
  double staged_gather_gbps;    /* staged path: device-side gather/scatter rate */
  double kernel_group_us[2];    /* gap per further kernel launch of one call */
  double staged_min_gain;       /* AUTO takes the staged path only if its modelled time is
                                   below (1 - staged_min_gain) x the best direct path's */
  double index_zero_copy_max_bytes[2]; /* kernel and staged paths: a request whose index
                                   pairs (16 bytes per position) fit in this many bytes
                                   has them read by the kernels from the mapped pinned
                                   staging buffer, skipping the copy to the device */
  double duplex_kernel_max_workgroups[2]; /* kernel-path grid cap while the other
                                   direction is busy ([0] backup, [1] load; 0 = none) */
  double kernel_wg_gbps[2];     /* kernel path: bytes one workgroup moves per second (GB/s) */
  double kernel_wg_row_ns[2];   /* kernel path: a workgroup's extra time per row (ns) */
  double kernel_wg_start_bytes[2]; /* capped kernel grid: bytes at the start of a call
                                      that move more slowly (0 = none) */
  double kernel_wg_start_us[2]; /* capped kernel grid: what those bytes cost in full (us) */
  double kernel_link_gap_us[2]; /* kernel path: link idle time per further launch (us) */
  double kernel_pace_gbps[2];   /* kernel and LDS paths: > 0 paces a capped launch's
                                   workgroups to this total rate (GB/s, >= 1) on the
                                   device's wall clock; 0 = unpaced */
  double kernel_pace_burst_blocks[2]; /* paced launches: blocks each workgroup moves at
                                   once before its pacing starts (whole number, 0..2^16) */
  double kernel_wg_jump_ns[2];  /* kernel path: a workgroup's extra time per walk row whose
                                   device row does not follow the previous one's (ns) */
  double kernel_cu_exclusive[2]; /* kernel path, a launch under a grid cap (a write-back's,
                                   an overlapped load's, a duplex one): 1 = each workgroup
                                   asks for a compute unit's whole LDS, so that no other
                                   kernel's workgroups share its compute units; 0 = off */
  double kernel_lane_depth[2];  /* kernel path: 8-byte chunks each lane keeps in flight,
                                   1, 2, 4 or 8. A workgroup's rate grows with it (a
                                   write-back workgroup ~3.3 GB/s at 2, ~6.6 at 8); at a
                                   given rate, more workgroups with fewer accesses in flight
                                   each cost a kernel beside them less. Defaults 2 for a
                                   backup, 8 for a load; kernel_wg_gbps and the slow start
                                   are fitted at the default */
} kv_calib_t;

typedef struct kv_pool kv_pool_t; /* opaque */

/* ---- planner: pure host functions, no GPU needed ------------------------ */

/* Checks a geometry: L,C,ps >= 1, R >= 16 and R % 16 == 0, S_dev,S_host >= 1,
 * S_host % ps == 0, layout in range, and the pool sizes fit in int64.
 * Returns KV_OK or KV_EINVAL. */
int kv_geometry_check(const kv_geometry_t *geom);

/* Host row index of (layer, comp, host slot) in the pool's layout (formulas
 * above). Returns the row (>= 0) or KV_EINVAL / KV_ERANGE for a bad geometry
 * or out-of-range argument. Byte offset = row * R. */
int64_t kv_host_row(const kv_geometry_t *geom, int32_t layer, int32_t comp, int64_t host_slot);

/* Validates one transfer exactly as kv_backup (direction 0) / kv_load
 * (direction 1) do before enqueuing anything:
 *   KV_EINVAL  null index pointer with n > 0, n < 0, or not
 *              0 <= layer_begin <= layer_end <= L;
 *   KV_ERANGE  some dev_idx[i] outside [0,S_dev) or host_idx[i] outside [0,S_host);
 *   KV_EDUP    (check_unique != 0) a destination slot repeats: host_idx for
 *              backup, dev_idx for load; the message names the first position
 *              whose slot appeared earlier in the request.
 * The first failing rule in this order decides the code. n == 0 is KV_OK.
 * The duplicate check costs O(n) with a per-slot table while the pool has at
 * most max(2^22, 4n) destination slots, else O(n log n) on a sorted copy. */
int kv_validate(const kv_geometry_t *geom, int32_t direction, const int64_t *dev_idx,
                const int64_t *host_idx, int64_t n, int32_t layer_begin, int32_t layer_end,
                int32_t check_unique);

/* Number of contiguous copies ("DMA segments") the request needs: for each
 * (l in [layer_begin,layer_end), c), the maximal runs of consecutive request
 * positions whose device rows and host rows both advance by exactly one row.
 * Runs never cross (l,c) buffers. This is the segment count of the Kunlunxin
 * tuning page section 2.1: page_num*layer_num for page_first_direct against
 * layer_num for layer_first at C = 1. Validates first (as kv_validate with
 * check_unique = 0); *out is written only on KV_OK. */
int kv_count_segments(const kv_geometry_t *geom, const int64_t *dev_idx, const int64_t *host_idx,
                      int64_t n, int32_t layer_begin, int32_t layer_end, int64_t *out);

/* Number of copy-engine calls the DMA path would issue for the request after
 * merging equal-length runs at a uniform device and host stride into 2-D copies.
 * A 2-D call names pitch x lines bytes on each side; where that region would
 * end past the host pool or the device buffer (the last line itself always
 * fits), the last line goes out as a 1-D call of its own, and is counted so.
 * Validates like kv_count_segments. */
int kv_count_dma_copies(const kv_geometry_t *geom, const int64_t *dev_idx,
                        const int64_t *host_idx, int64_t n, int32_t layer_begin,
                        int32_t layer_end, int64_t *out);

/* ---- pool lifetime (needs a GPU) ----------------------------------------- */

/* Allocates the pinned, device-mapped host pool (L*C*S_host*R bytes, contents
 * unspecified), copies the device-buffer table to the device, creates the
 * per-layer load events and the per-direction index staging buffers. The
 * host pool is pinned once, up front, and optionally bound to the GPU's NUMA
 * node (numa_node) or interleaved (KV_F_HOST_INTERLEAVE): the pages tie
 * host-link throughput to pinned, registered host memory and to its NUMA
 * placement ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.4
 * "The physical form of Host memory"; "Baidu's KVCache Overhaul", "Host Memory
 * & Link Optimization").
 * Not on the timed path. On success *out owns all of it. Errors: KV_EINVAL
 * (bad desc / geometry / null buffer / misaligned buffer), KV_ENOMEM,
 * KV_EHIP. */
int kv_pool_create(const kv_pool_desc_t *desc, kv_pool_t **out);

/* Creates a pool over its own device buffers that SHARES the host pool of
 * `group` (any pool made by kv_pool_create, or by this call from one), instead
 * of allocating one: the tensor-parallel group's shared host KV buffer
 * ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.7, "TP group
 * shared Host KV"; "Baidu's KVCache Overhaul", "TP-group shared host KV
 * buffer"). Where every rank holds bit-identical KV (a replicated MLA latent),
 * one host copy serves the group: the pool made by kv_pool_create (the
 * writer) does the write-back, every pool of the group loads from the same
 * host bytes with its own indices into its own device buffers.
 *   - desc->geom must equal the writer's except device_slots; desc->device
 *     may name another device (the host pool is allocated portable and mapped);
 *     desc->numa_node and KV_F_HOST_NONCOHERENT are ignored (the host memory is
 *     the writer's); the other flags apply to this pool.
 *   - kv_backup on a sharing pool moves no data. It validates the request as a
 *     backup would (same error codes), then makes `stream` wait for the
 *     writer's most recent backup: the rank still reports completion through
 *     its own stream, and that completion is gated by the writer's write. Call
 *     it after the writer's matching backup has been enqueued. With
 *     KV_F_SHARE_CHECK on the writer, a request whose host slots or layer
 *     range differ from the writer's most recent backup is refused (KV_EINVAL):
 *     the group's host allocation must be the same on every rank.
 *     kv_last_path then reports KV_PATH_SHARED and no bytes are counted.
 *   - kv_load on a sharing pool is an ordinary load from the shared host pool.
 *   - The host pool lives until every pool of the group is destroyed, in any
 *     order.
 * Errors: KV_EINVAL (null group/desc/out, geometry differing from the
 * writer's, bad device buffers), KV_ENOMEM, KV_EHIP. */
int kv_pool_create_shared(const kv_pool_desc_t *desc, kv_pool_t *group, kv_pool_t **out);

/* Waits for every transfer enqueued through the pool, then frees its events
 * and staging, and the host pool once no pool of its group uses it. Returns
 * the first HIP error seen while waiting, if any. NULL is a no-op returning
 * KV_OK. */
int kv_pool_destroy(kv_pool_t *pool);

/* Host (CPU) address of the host pool and its size in bytes. The pointer stays
 * valid until kv_pool_destroy. Reading it while a transfer that writes it is
 * in flight gives unspecified bytes. */
void *kv_pool_host_ptr(const kv_pool_t *pool);
int64_t kv_pool_host_bytes(const kv_pool_t *pool);

/* ---- transfers (the hot path) -------------------------------------------- */

/* D2H write-back: for every i in [0,n), l in [layer_begin,layer_end), c in
 * [0,C), copy the R bytes of device row dev_idx[i] of B[l][c] to host row
 * host_row(l,c,host_idx[i]). Enqueued on `stream` (a hipStream_t; NULL = the
 * null stream). dev_idx/host_idx are host arrays of n int64, read only during
 * the call. The caller orders `stream` after the work that produced the KV and
 * must not overwrite those device rows until the stream has passed this call.
 * Returns after enqueue. n == 0 or an empty layer range: KV_OK, nothing
 * enqueued. */
int kv_backup(kv_pool_t *pool, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
              int32_t layer_begin, int32_t layer_end, void *stream);

/* H2D load: the reverse copy, host row host_row(l,c,host_idx[i]) -> device row
 * dev_idx[i] of B[l][c]. Layers are issued in increasing order, in groups
 * (see load_split_min_bytes), and after each group a landed event is recorded
 * on `stream`, so a consumer can start on layer l while later layers are
 * still in flight (compute/transfer overlap: HiCache system design page,
 * "data transfer optimisation"; the load stream signalling a per-layer ready
 * event that the compute stream waits on: runtime-boundary page, "why
 * compute, H2D and D2H should stay in one GPU execution domain"). On the
 * staged path a page_first / page_first_direct load is one group: every layer
 * lands at its end (AUTO leaves that path out under KV_F_LOAD_OVERLAP). The
 * caller must not overwrite those host rows until the load has completed. */
int kv_load(kv_pool_t *pool, const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
            int32_t layer_begin, int32_t layer_end, void *stream);

/* kv_backup (direction 0) or kv_load (direction 1) that allocates nothing, for
 * callers that cannot allocate device or pinned memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. It always
 * takes the zero-copy kernel path (KV_PATH_KERNEL; kv_last_path reports it),
 * with that path's grid caps, load groups and landed events, so kv_load_layer
 * works after it as after kv_load. Instead of the pool's index staging, the
 * request's index arrays are copied from the caller's host arrays into a
 * device array the library holds for each GPU from its first such call until
 * the process ends. A pageable array is read before the call returns (the
 * runtime stages it); a page-locked one is read by the copy on `stream`, so
 * the caller keeps it unchanged until the stream has passed the call. The
 * device array holds 8 MiB: n <= 262144 positions
 * (a larger n: KV_EINVAL, nothing enqueued). The index pairs are formed there
 * on the device. Every call on one GPU shares that GPU's array: calls issued on
 * one stream are ordered, but calls that overlap on one GPU (other streams,
 * or other threads without ordering) race and may move the wrong rows. With
 * KV_F_CHECK_UNIQUE the destination check uses the per-slot table kv_pool_create
 * sizes for pools of up to 2^24 destination slots (4 bytes per slot); a larger
 * pool's table exists only once a kv_backup / kv_load of that direction has
 * sized it, else the call returns KV_EINVAL. On
 * success the call allocates nothing; a failure's message may. Errors as
 * kv_backup / kv_load, and KV_EINVAL for a direction other than 0 or 1. */
int kv_transfer_noalloc(kv_pool_t *pool, int32_t direction, const int64_t *dev_idx,
                        const int64_t *host_idx, int64_t n, int32_t layer_begin,
                        int32_t layer_end, void *stream);

/* The staged path's device-side pass on its own: the batched gather/scatter
 * that packs a request's scattered device rows into one contiguous,
 * host-ordered buffer in HBM, so that a single large copy moves it ("Baidu's
 * KVCache Overhaul", "DMA Segment Explosion & Batched Gather/Scatter").
 * direction 0 packs the rows of positions [0, n), layers [layer_begin,
 * layer_end), from the device buffers into `stage`; direction 1 unpacks them
 * from `stage` into the device buffers. Row order in `stage` is the host
 * address order of the pool's layout, as if the request's positions were host
 * slots 0..n-1 of a pool holding layers [layer_begin, layer_end) only:
 *   layer_first        (layer, comp, position)
 *   page_first         (position, layer, comp)
 *   page_first_direct  (page of ps positions, layer, comp, position in page);
 *                      the last page holds the n % ps positions left, if any.
 * So a request on whole, consecutive host pages packs into exactly the bytes
 * the host pool holds for those pages, and one copy moves them to L2 or to an
 * L3 store. `stage`: device memory of the pool's device, 16-byte aligned,
 * n * (layer_end - layer_begin) * C * R bytes, BORROWED until the stream has
 * passed the call. dev_idx: host array of n int64, read during the call.
 * Enqueued on `stream`; the caller orders it after the work that produced the
 * rows (pack) or the stage's bytes (unpack). Errors as kv_backup (KV_EDUP only
 * for an unpack, with KV_F_CHECK_UNIQUE); KV_EINVAL also for a direction other
 * than 0 or 1 and for a stage that is null, misaligned, not device memory of
 * the pool's device, or whose rows would run past the end of the device
 * allocation holding it (a buffer carved out of a larger allocation, as a
 * caching allocator hands out, is checked against that allocation only).
 * n == 0 or an empty layer range: KV_OK, nothing enqueued. */
int kv_stage(kv_pool_t *pool, int32_t direction, const int64_t *dev_idx, int64_t n,
             int32_t layer_begin, int32_t layer_end, void *stage, void *stream);

/* Makes `compute_stream` wait (on the device, the host does not block) until
 * layer `layer` of the most recent kv_load that covered that layer on this
 * pool has landed in device memory: the load stream signals a per-layer ready
 * event and the compute stream waits on it, so compute, H2D and D2H stay in one
 * GPU execution domain ordered by events ("Rethinking the SGLang HiCache
 * Boundary: From L2 Offload to a Cache Runtime", section "Why compute, H2D, and
 * D2H should stay in one GPU execution domain"). Call it after that kv_load has
 * returned. The wait is on the landed event of the layer's group in that load
 * (see load_split_min_bytes), so it may also cover the other layers of that
 * group. Each group records an event of its own, and an event is recorded
 * again only once no layer names it and its previous recording has
 * completed, so the wait never covers less than the layer asked for, whatever
 * later loads on other streams cover. A layer no kv_load has covered yet:
 * KV_OK, no wait. After a kv_load that returned an error, which of its layers
 * were enqueued is unspecified, and so is this wait for them. Errors:
 * KV_EINVAL (layer out of [0,L)), KV_EHIP. */
int kv_load_layer(kv_pool_t *pool, int32_t layer, void *compute_stream);

/* ---- streams -------------------------------------------------------------- */

/* Creates a HIP stream (returned as hipStream_t in *out) on `device` that has a
 * hardware queue of its own. The runtime maps ordinary streams onto a few
 * hardware queues round-robin; two streams on one queue run in order, so a
 * backup stream and a load stream that share a queue cannot use both link
 * directions at once, and a load stream that shares the compute stream's queue
 * cannot overlap compute. Streams from this call never share a queue (they
 * carry a CU mask that enables every compute unit, which gives them their own
 * queue without restricting where kernels run). Default priority. The caller
 * owns the stream and destroys it with kv_stream_destroy. Errors: KV_EINVAL,
 * KV_EHIP. */
int kv_stream_create(int32_t device, void **out);

/* Waits for the stream's work and destroys it. NULL is a no-op. */
int kv_stream_destroy(void *stream);

/* ---- path control, calibration and statistics -------------------------- */

/* Forces a path (kv_path_t) for later calls on this pool, both directions;
 * KV_PATH_AUTO restores the selector. */
int kv_set_path(kv_pool_t *pool, int32_t path);

/* The same for one direction only (0 = backup, 1 = load), e.g. write-backs on
 * the staged path while loads stay on the kernel path, the pairing the
 * bidirectional mixed batch runs with a dedicated thread and stream per
 * direction ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.2;
 * "Baidu's KVCache Overhaul", "Bidirectional Async Transfer"). Errors:
 * KV_EINVAL (null pool, bad direction or path). */
int kv_set_direction_path(kv_pool_t *pool, int32_t direction, int32_t path);

/* Path the most recent call of `direction` (0 = backup, 1 = load) used: one of
 * KV_PATH_KERNEL / KV_PATH_KERNEL_LDS / KV_PATH_DMA / KV_PATH_STAGED (or
 * KV_PATH_SHARED for the backup of a pool sharing another's host pool), or -1
 * if none yet. */
int32_t kv_last_path(const kv_pool_t *pool, int32_t direction);

/* Replaces / reads the selector calibration. */
int kv_set_calibration(kv_pool_t *pool, const kv_calib_t *calib);
int kv_get_calibration(const kv_pool_t *pool, kv_calib_t *calib);

/* Measures the pool's D2H host-link rate and paces the kernel path's
 * write-backs under it: kernel_pace_gbps[0] = fraction * the measured rate.
 * For callers that write back on the GPU-assisted kernel path (the zero-copy
 * kernels of the HiCache system design page, "data transfer optimisation")
 * beside compute, on a host whose link rate they do not know: the paced grid
 * must stay under what the link drains, which differs by host (see
 * kernel_pace_gbps). The rate is the median of 5 timed copy-engine copies (after
 * one untimed) of min(256 MiB, host pool, one device buffer) bytes from device
 * buffer 0 into the start of the host pool, on `stream`; the call blocks
 * until they finish (~30 ms). It OVERWRITES those host-pool bytes, so call it
 * before the pool holds data, and not within a second of the process freeing
 * gigabytes (the runtime's copies run slow then, which only lowers the pace).
 * The pool's transfers already in flight are waited for first, and its other
 * calls wait for the measurement. fraction in (0, 1]; 0.98 keeps the grid
 * under the link on the hosts measured. *d2h_gbps (may be null) receives the
 * measured rate. KV_EINVAL: null pool, fraction out of range, a pool that
 * shares another pool's host pool (calibrate the group's writer), a host pool
 * or first device buffer under 16 MiB, or a pace below 1 GB/s; KV_EHIP on a
 * runtime error (the calibration is then unchanged). */
int kv_calibrate_write_pace(kv_pool_t *pool, double fraction, void *stream, double *d2h_gbps);

typedef struct {
  int64_t calls[2];         /* per direction (0 backup, 1 load) */
  int64_t bytes[2];         /* algorithmic bytes enqueued */
  int64_t kernel_launches[2];
  int64_t dma_copies[2];    /* copy-engine calls issued */
  double submit_us[2];      /* host wall time spent inside the calls, minus blocked_us */
  double blocked_us[2];     /* host time spent waiting for an index staging buffer
                               (only when 16 calls of one direction are in flight) or,
                               for loads, for a free landed event (only when more
                               than L + 16 load groups are in flight) */
  int64_t last_workgroups[2]; /* grid of the latest launch of a kernel that moves rows
                               (direct or LDS kernel, or the staged path's device-side
                               pass, kv_stage's included), after any cap; 0 before
                               the first */
} kv_stats_t;

int kv_get_stats(const kv_pool_t *pool, kv_stats_t *out);

/* The library's default calibration (the figures a new pool starts with). */
int kv_default_calibration(kv_calib_t *calib);

/* The path selector without a GPU: for a request as kv_backup (direction 0)
 * or kv_load (1) would get it on a pool of this geometry and calibration,
 * writes the modelled times of the kernel, copy-engine and staged paths to
 * times_us[0..2] (microseconds; the staged one may be +infinity where AUTO
 * leaves that path out) and returns the path AUTO takes (KV_PATH_KERNEL,
 * KV_PATH_DMA or KV_PATH_STAGED). flags: KV_F_LOAD_OVERLAP as on a pool;
 * KV_F_DUPLEX stands for the other direction being busy. The request is
 * validated as kv_validate does without the uniqueness check; an empty
 * request, a bad argument or calibration: KV_EINVAL (or the validation code). */
int32_t kv_model_path(const kv_geometry_t *geom, const kv_calib_t *calib, int32_t direction,
                      const int64_t *dev_idx, const int64_t *host_idx, int64_t n,
                      int32_t layer_begin, int32_t layer_end, uint32_t flags,
                      double *times_us);

/* Message describing the last failure on the calling thread ("" if none). */
const char *kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVTIER_H */
