"""GPU parity: the C-ABI transfers against the oracle, byte for byte.

Small pools whose requests span many workgroups, LDS tiles and copy-engine
copies, with ragged tails (request sizes that are not a multiple of the page
size, row sizes that are not a power of two), every host layout, every path,
both directions, partial layer ranges, and the edge cases (empty requests,
empty layer ranges, one-token requests, 16-byte rows, rejected requests).
"""
import itertools

import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
from hierarchical_kv_cache_backup_amd import workloads
import oracle
from oracle import Geometry, LAYOUTS, np_ref

from gpu_util import (PATHS, SENTINEL, device_buffers, make_pool, mirrors,
                      run_backup_and_compare, run_load_and_compare, kv_geom, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture
def stream(torch):
    return torch.cuda.Stream()


# ---- config 1: tiny pool, round trip into fresh slots ------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("path", PATHS)
def test_tiny_round_trip(torch, stream, layout, path):
    shape = workloads.tiny()
    g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                 shape.host_slots, shape.page_size, layout)
    dev_idx, host_idx, reload_idx = workloads.tiny_indices(shape)
    src = device_buffers(g, seed=1)
    pool = make_pool(g, src, path)
    print("tiny layout=%d path=%d" % (layout, path), flush=True)
    run_backup_and_compare(g, pool, src, dev_idx, host_idx, 0, g.L, stream)
    # reload into a second, sentinel-filled device pool at an independent permutation
    fresh = device_buffers(g, seed=2, fill=SENTINEL)
    pool2 = make_pool(g, fresh, path, host_fill=None)
    pool2.host_array()[:] = pool.host_array()
    run_load_and_compare(g, pool2, fresh, reload_idx, host_idx, 0, g.L, stream)
    # identity: fresh[reload[i]] == src[dev[i]] for every row
    for k in range(g.L * g.C):
        a = src[k].view(g.S_dev, g.R)[torch.from_numpy(dev_idx).cuda()]
        b = fresh[k].view(g.S_dev, g.R)[torch.from_numpy(reload_idx).cuda()]
        assert torch.equal(a, b)
    pool.close()
    pool2.close()


# ---- random requests over several tiles with ragged tails ----------------------------

GEOMS = [
    # L, C, R, S_dev, S_host, ps
    (3, 2, 272, 700, 640, 16),
    (5, 1, 1152, 300, 256, 64),
    (2, 2, 16, 2000, 2048, 4),
    (4, 2, 2048, 200, 192, 64),
]


def _request(rng, g, kind):
    n = int(min(g.S_dev, g.S_host) * 0.8) + 3
    n = min(n, g.S_dev, g.S_host)
    if kind == "random":
        return (rng.choice(g.S_dev, n, replace=False).astype(np.int64),
                rng.choice(g.S_host, n, replace=False).astype(np.int64))
    if kind == "contiguous":
        d0 = int(rng.integers(0, g.S_dev - n + 1))
        return np.arange(d0, d0 + n, dtype=np.int64), np.arange(n, dtype=np.int64)
    # whole device pages in random order, host slots in order
    pages = rng.permutation(g.S_dev // g.ps)[: n // g.ps]
    d = workloads.page_indices(pages, g.ps)
    return d.astype(np.int64), np.arange(d.size, dtype=np.int64)


@pytest.mark.parametrize("gi", range(len(GEOMS)))
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("path", PATHS)
def test_random_requests_match_oracle(torch, stream, gi, layout, path):
    L, C, R, S_dev, S_host, ps = GEOMS[gi]
    g = Geometry(L, C, R, S_dev, S_host, ps, layout)
    rng = np.random.default_rng(100 * gi + 10 * layout + path)
    bufs = device_buffers(g, seed=gi)
    pool = make_pool(g, bufs, path)
    for kind in ("random", "contiguous", "pages"):
        d, h = _request(rng, g, kind)
        for l0, l1 in ((0, L), (1, L), (0, 1)):
            print("geom=%d layout=%d path=%d kind=%s layers=[%d,%d) n=%d" %
                  (gi, layout, path, kind, l0, l1, d.size), flush=True)
            run_backup_and_compare(g, pool, bufs, d, h, l0, l1, stream)
            pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            run_load_and_compare(g, pool, bufs, d, h, l0, l1, stream)
            assert pool.last_path(kvt.LOAD) in (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS, kvt.PATH_DMA,
                                                kvt.PATH_STAGED)
            if path != kvt.PATH_AUTO:
                assert pool.last_path(kvt.BACKUP) == path
    pool.close()


# ---- edge cases --------------------------------------------------------------------

def test_edge_cases(torch, stream):
    g = Geometry(2, 2, 16, 64, 64, 8, oracle.PAGE_FIRST_DIRECT)
    bufs = device_buffers(g, seed=5)
    for path in PATHS:
        pool = make_pool(g, bufs, path)
        before = pool.host_array().copy()
        # empty request / empty layer range: OK, nothing moves
        pool.backup([], [], 0, 2, stream)
        pool.backup([1, 2], [3, 4], 1, 1, stream)
        stream.synchronize()
        assert np.array_equal(pool.host_array(), before)
        # one token, last slots
        run_backup_and_compare(g, pool, bufs, [63], [63], 0, 2, stream)
        run_load_and_compare(g, pool, bufs, [0], [63], 1, 2, stream)
        # whole pool
        run_backup_and_compare(g, pool, bufs, np.arange(64)[::-1], np.arange(64), 0, 2, stream)
        # rejected requests change nothing
        snap = pool.host_array().copy()
        dev_snap = [b.clone() for b in bufs]
        cases = [(kvt.EDUP, "backup", [1, 2], [5, 5], 0, 2),
                 (kvt.ERANGE, "backup", [64], [0], 0, 2),
                 (kvt.ERANGE, "load", [0], [-1], 0, 2),
                 (kvt.EINVAL, "load", [0], [0], 0, 3),
                 (kvt.EINVAL, "backup", [0], [0], 2, 1),
                 (kvt.EDUP, "load", [7, 7], [1, 2], 0, 2)]
        for code, op, d, h, l0, l1 in cases:
            fn = kvt.kv_backup if op == "backup" else kvt.kv_load
            rc = fn(pool.handle, d, h, l0, l1, stream)
            assert rc == code, (op, d, h, l0, l1, rc, kvt.kv_last_error())
            assert kvt.kv_last_error()
        assert kvt.kv_backup(pool.handle, [1], [1], 0, 2, stream, n=-1) == kvt.EINVAL
        stream.synchronize()
        assert np.array_equal(pool.host_array(), snap)
        for a, b in zip(bufs, dev_snap):
            assert torch.equal(a, b)
        assert kvt.kv_load_layer(pool.handle, 2, stream) == kvt.EINVAL
        assert kvt.kv_load_layer(pool.handle, -1, stream) == kvt.EINVAL
        assert kvt.kv_set_path(pool.handle, 7) == kvt.EINVAL
        assert kvt.kv_set_path(pool.handle, -1) == kvt.EINVAL
        pool.close()
    # duplicates are accepted when the pool does not check them (last writer unspecified,
    # so only a non-overlapping request is compared)
    pool = make_pool(g, bufs, kvt.PATH_KERNEL, flags=0)
    assert kvt.kv_backup(pool.handle, [1, 2], [5, 5], 0, 2, stream) == kvt.OK
    stream.synchronize()
    pool.close()


def test_pool_create_rejects_bad_buffers(torch):
    g = Geometry(1, 2, 32, 16, 16, 4, 0)
    good = device_buffers(g, seed=0)
    kg = kv_geom(g)
    # a buffer that runs 16 bytes past the end of its device allocation (torch's
    # caching allocator sub-allocates, so find the end of the real segment)
    holder = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    seg_end = None
    for seg in torch.cuda.memory_snapshot():
        if seg["address"] <= holder.data_ptr() < seg["address"] + seg["total_size"]:
            seg_end = seg["address"] + seg["total_size"]
    assert seg_end is not None
    over = seg_end - g.S_dev * g.R + 16
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), over])
    assert rc == kvt.EINVAL and h is None, kvt.kv_last_error()
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), over - 16])
    assert rc == kvt.OK, kvt.kv_last_error()
    assert kvt.kv_pool_destroy(h) == kvt.OK
    big = torch.zeros(16 * 32 + 16, dtype=torch.uint8, device="cuda:0")
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), big.data_ptr() + 8])
    assert rc == kvt.EINVAL
    cpu = np.zeros(16 * 32, np.uint8)
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), cpu.ctypes.data])
    assert rc == kvt.EINVAL
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), good[1].data_ptr()], device=99)
    assert rc == kvt.EINVAL
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), good[1].data_ptr()], numa_node=4096)
    assert rc == kvt.EINVAL
    bad = kvt.geometry(1, 2, 24, 16, 16, 4, 0)
    rc, h = kvt.kv_pool_create(bad, [good[0].data_ptr(), good[1].data_ptr()])
    assert rc == kvt.EINVAL
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), good[1].data_ptr()], numa_node=0,
                               flags=kvt.F_CHECK_UNIQUE | kvt.F_HOST_NONCOHERENT)
    assert rc == kvt.OK, kvt.kv_last_error()
    assert kvt.kv_pool_host_bytes(h) == 2 * 16 * 32
    assert kvt.kv_pool_destroy(h) == kvt.OK
    assert kvt.kv_pool_destroy(None) == kvt.OK
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), good[1].data_ptr()], numa_node=64)
    assert rc == kvt.EINVAL
    rc, h = kvt.kv_pool_create(kg, [good[0].data_ptr(), good[1].data_ptr()], numa_node=0,
                               flags=kvt.F_CHECK_UNIQUE | kvt.F_HOST_INTERLEAVE)
    assert rc == kvt.EINVAL and "exclusive" in kvt.kv_last_error()


def test_interleaved_host_pool_parity(torch, stream):
    """A host pool spread over every online NUMA node moves the same bytes."""
    g = Geometry(3, 2, 272, 700, 640, 16, oracle.PAGE_FIRST_DIRECT)
    bufs = device_buffers(g, seed=19)
    rng = np.random.default_rng(19)
    for path in (kvt.PATH_KERNEL, kvt.PATH_DMA):
        pool = make_pool(g, bufs, path, flags=kvt.F_CHECK_UNIQUE | kvt.F_HOST_INTERLEAVE)
        d, h = _request(rng, g, "random")
        run_backup_and_compare(g, pool, bufs, d, h, 0, 3, stream)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, 0, 3, stream)
        pool.close()


def test_noncoherent_host_pool_parity(torch, stream):
    g = Geometry(3, 2, 272, 700, 640, 16, oracle.PAGE_FIRST)
    bufs = device_buffers(g, seed=9)
    rng = np.random.default_rng(9)
    for path in (kvt.PATH_KERNEL, kvt.PATH_DMA):
        pool = make_pool(g, bufs, path, flags=kvt.F_CHECK_UNIQUE | kvt.F_HOST_NONCOHERENT)
        d, h = _request(rng, g, "random")
        run_backup_and_compare(g, pool, bufs, d, h, 0, 3, stream)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, 0, 3, stream)
        pool.close()


def test_stats_and_calibration(torch, stream):
    g = Geometry(2, 1, 64, 32, 32, 8, 0)
    bufs = device_buffers(g, seed=3)
    pool = make_pool(g, bufs, kvt.PATH_AUTO)
    c = pool.calibration()
    assert c.kernel_gbps[0] > 0 and c.load_split_min_bytes >= 0
    # a calibration that makes copies free selects the copy engines
    c.dma_copy_us[0] = 0.0
    c.dma_gbps[0] = 1e6
    pool.set_calibration(c)
    pool.backup(np.arange(8), np.arange(8), 0, 2, stream)
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_DMA
    c.dma_copy_us[0] = 1e6
    pool.set_calibration(c)
    pool.backup(np.arange(8), np.arange(8), 0, 2, stream)
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_KERNEL
    stream.synchronize()
    s = pool.stats()
    assert s.calls[0] == 2 and s.bytes[0] == 2 * 8 * 2 * 64
    assert s.kernel_launches[0] == 1 and s.dma_copies[0] == 2
    c.kernel_gbps[0] = -1
    with pytest.raises(kvt.KvError):
        pool.set_calibration(c)
    pool.close()


# ---- capped grids: workgroups stride over many blocks of work ------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
def test_capped_grid_matches_oracle(torch, stream, layout):
    L, C, R, S_dev, S_host, ps = GEOMS[0]
    g = Geometry(L, C, R, S_dev, S_host, ps, layout)
    bufs = device_buffers(g, seed=11)
    rng = np.random.default_rng(11 + layout)
    for path in (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS):
        pool = make_pool(g, bufs, path)
        # capped grids with and without a compute unit per workgroup
        # (kernel_cu_exclusive), each way, at every lane depth; and full grids
        # (cap 0) at the shallow depths
        for cap, excl, depth in ((1, 1, 8), (3, 0, 2), (7, 1, 4), (7, 0, 1), (0, 0, 1),
                                 (0, 0, 2)):
            c = pool.calibration()
            c.kernel_max_workgroups[0] = c.kernel_max_workgroups[1] = cap
            c.kernel_cu_exclusive[0] = c.kernel_cu_exclusive[1] = excl
            c.kernel_lane_depth[0] = c.kernel_lane_depth[1] = depth
            pool.set_calibration(c)
            d, h = _request(rng, g, "random")
            print("capped layout=%d path=%d cap=%d exclusive=%d depth=%d"
                  % (layout, path, cap, excl, depth), flush=True)
            run_backup_and_compare(g, pool, bufs, d, h, 0, L, stream)
            pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            run_load_and_compare(g, pool, bufs, d, h, 0, L, stream)
        pool.close()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_paced_grid_matches_oracle(torch, stream, layout):
    """kernel_pace_gbps holds a capped kernel grid to a set rate: the bytes of a
    paced backup and load (kv_backup / kv_load and kv_transfer_noalloc) match
    the oracle, and each call takes at least what the pace allows: after its
    first max(1, burst) blocks a workgroup starts its blocks of rows_per_block
    rows at least grid * block bytes / rate apart, with one block of catch-up,
    so the busiest workgroup's m blocks take at least m - max(1, burst) - 1
    such intervals."""
    L, C, R, S_dev, S_host, ps = GEOMS[1]
    g = Geometry(L, C, R, S_dev, S_host, ps, layout)
    bufs = device_buffers(g, seed=12)
    rng = np.random.default_rng(12 + layout)
    pool = make_pool(g, bufs, kvt.PATH_KERNEL)
    cap, gbps, burst = 3, 1.0, 4
    c = pool.calibration()
    assert list(c.kernel_pace_gbps) == [54.0, 0.0]     # defaults: backups paced, loads not
    assert list(c.kernel_pace_burst_blocks) == [32.0, 0.0]
    c.kernel_max_workgroups[:] = [cap, cap]
    c.kernel_pace_gbps[:] = [gbps, gbps]
    c.kernel_pace_burst_blocks[:] = [burst, burst]
    pool.set_calibration(c)
    rows_per_block = 2048 // (R // 8)            # 16 KiB of 8-byte chunks per block
    interval_s = cap * rows_per_block * R / (gbps * 1e9)
    launches = list(pool.stats().kernel_launches)
    for noalloc in (False, True):
        d, h = _request(rng, g, "random")
        n = len(d)
        print("paced layout=%d noalloc=%d n=%d" % (layout, noalloc, n), flush=True)
        # one launch each way: a backup is one group, and a load this small too
        blocks = -(-n * L * C // rows_per_block)
        floor_s = max(0, -(-blocks // cap) - max(1, burst) - 1) * interval_s
        for direction in (kvt.BACKUP, kvt.LOAD):
            want_host = pool.host_array().copy()
            dev_m = mirrors(bufs)
            if direction == kvt.BACKUP:
                assert oracle.backup(g, dev_m, want_host, d, h, 0, L) == 0
            else:
                pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
                want_host = pool.host_array().copy()
                assert oracle.load(g, dev_m, want_host, d, h, 0, L) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if noalloc:
                rc = kvt.kv_transfer_noalloc(pool.handle, direction, d, h, 0, L, stream)
                assert rc == kvt.OK, kvt.kv_last_error()
            elif direction == kvt.BACKUP:
                pool.backup(d, h, 0, L, stream)
            else:
                pool.load(d, h, 0, L, stream)
            e1.record(stream)
            stream.synchronize()
            torch.cuda.synchronize()
            assert pool.stats().last_workgroups[direction] == cap
            assert np.array_equal(pool.host_array(), want_host)
            for k, b in enumerate(bufs):
                assert np.array_equal(b.cpu().numpy(), dev_m[k]), k
            took = e0.elapsed_time(e1) / 1e3
            assert pool.stats().kernel_launches[direction] == launches[direction] + 1
            launches[direction] += 1
            assert took >= floor_s, (took, floor_s)
    for field, bad in (("kernel_pace_gbps", 0.5), ("kernel_pace_burst_blocks", 1.5),
                       ("kernel_pace_burst_blocks", -1.0), ("kernel_pace_burst_blocks", 65537.0)):
        c = pool.calibration()
        getattr(c, field)[0] = bad
        with pytest.raises(kvt.KvError):
            pool.set_calibration(c)
    pool.close()


def test_calibrate_write_pace(torch, stream):
    """kv_calibrate_write_pace times copies of device buffer 0 into the host
    pool and sets kernel_pace_gbps[0] to the given fraction of the median rate,
    leaving the rest of the calibration alone; the pool still moves bytes that
    match the oracle afterwards. It refuses fractions outside (0, 1], pools
    whose host pool or first buffer is under 16 MiB, and a pool that shares
    another pool's host pool."""
    g = Geometry(2, 1, 4096, 8192, 8192, 64, 0)     # 32 MiB buffers, 64 MiB host pool
    bufs = device_buffers(g, seed=23)
    pool = make_pool(g, bufs, kvt.PATH_KERNEL)
    before = pool.calibration()
    print("calibrate write pace", flush=True)
    gbps = pool.calibrate_write_pace(0.9, stream)
    assert 1.0 < gbps < 200.0, gbps
    c = pool.calibration()
    assert c.kernel_pace_gbps[0] == pytest.approx(0.9 * gbps)
    assert c.kernel_pace_gbps[1] == before.kernel_pace_gbps[1]
    assert list(c.kernel_max_workgroups) == list(before.kernel_max_workgroups)
    assert list(c.dma_gbps) == list(before.dma_gbps)
    # the measurement wrote the start of the host pool; transfers stay exact
    rng = np.random.default_rng(23)
    pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
    d = rng.permutation(g.S_dev)[:6000].astype(np.int64)
    h = rng.permutation(g.S_host)[:6000].astype(np.int64)
    run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
    for bad in (0.0, -0.5, 1.5, float("nan")):
        rc, _ = kvt.kv_calibrate_write_pace(pool.handle, bad, stream)
        assert rc == kvt.EINVAL, bad
    assert pool.calibration().kernel_pace_gbps[0] == pytest.approx(0.9 * gbps)
    gs = Geometry(2, 1, 4096, 1024, 1024, 64, 0)    # 4 MiB buffers
    small = make_pool(gs, device_buffers(gs, seed=24))
    rc, _ = kvt.kv_calibrate_write_pace(small.handle, 0.98, stream)
    assert rc == kvt.EINVAL and "16 MiB" in kvt.kv_last_error()
    small.close()
    reader = kvt.KvPool(kv_geom(g), device_buffers(g, seed=25), share_with=pool)
    rc, _ = kvt.kv_calibrate_write_pace(reader.handle, 0.98, stream)
    assert rc == kvt.EINVAL and "writer" in kvt.kv_last_error()
    reader.close()
    pool.close()


def test_duplex_and_overlap_caps_bound_the_grid(torch, stream):
    """A backup's kernel launches at most kernel_max_workgroups[0] workgroups
    (default 18); the kernel paths launch at most duplex_kernel_max_workgroups[dir]
    on a KV_F_DUPLEX pool (defaults: 8 for a backup, 32 for a load), at most
    overlap_kernel_max_workgroups for a load flagged KV_F_LOAD_OVERLAP (default 24), and the
    smallest cap that applies; without a cap a launch has one workgroup per
    block of work. The bytes match the oracle under every cap."""
    g = Geometry(4, 2, 2048, 4096, 4096, 64, 0)
    bufs = device_buffers(g, seed=15)
    rng = np.random.default_rng(15)
    d = rng.permutation(g.S_dev).astype(np.int64)
    h = np.arange(g.S_host, dtype=np.int64)

    def grids(pool, path):
        pool.set_path(path)
        run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        return tuple(pool.stats().last_workgroups)

    plain = make_pool(g, bufs)
    c = plain.calibration()
    assert list(c.duplex_kernel_max_workgroups) == [8.0, 32.0]
    assert list(c.kernel_max_workgroups) == [18.0, 0.0]
    assert list(c.kernel_cu_exclusive) == [0.0, 1.0]
    assert list(c.kernel_lane_depth) == [2.0, 8.0]
    assert tuple(plain.stats().last_workgroups) == (0, 0)
    default = grids(plain, kvt.PATH_KERNEL)
    c.kernel_max_workgroups[0] = 0
    plain.set_calibration(c)
    free = grids(plain, kvt.PATH_KERNEL)
    assert free[0] > 1000 and free[1] > 1000, free     # one workgroup per 16 KiB block
    assert default == (18, free[1]), default
    c.duplex_kernel_max_workgroups[0] = -1
    with pytest.raises(kvt.KvError):
        plain.set_calibration(c)
    c = plain.calibration()
    c.kernel_cu_exclusive[1] = 0.5               # 0 or 1 only
    with pytest.raises(kvt.KvError):
        plain.set_calibration(c)
    for bad in (0.0, 3.0, 16.0):                 # 1, 2, 4 or 8 only
        c = plain.calibration()
        c.kernel_lane_depth[0] = bad
        with pytest.raises(kvt.KvError):
            plain.set_calibration(c)
    plain.close()

    duplex = make_pool(g, bufs, flags=kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX)
    assert grids(duplex, kvt.PATH_KERNEL) == (8, 32)
    lds = grids(duplex, kvt.PATH_KERNEL_LDS)
    assert 0 < lds[0] <= 8 and 0 < lds[1] <= 32, lds
    c = duplex.calibration()
    c.kernel_max_workgroups[:] = [0, 16]             # the tighter cap wins
    duplex.set_calibration(c)
    assert grids(duplex, kvt.PATH_KERNEL) == (8, 16)
    c.kernel_max_workgroups[:] = [0, 0]
    c.duplex_kernel_max_workgroups[:] = [0, 0]       # duplex caps off
    duplex.set_calibration(c)
    assert grids(duplex, kvt.PATH_KERNEL) == free
    duplex.close()

    overlap = make_pool(g, bufs, flags=kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP)
    got = grids(overlap, kvt.PATH_KERNEL)
    assert got == (18, 24), got                     # the overlap cap is a load's only
    overlap.close()


@pytest.mark.parametrize("R", (256, 512, 1152))
def test_staged_pass_on_a_capped_grid(torch, stream, R):
    """A load flagged KV_F_LOAD_OVERLAP runs the staged path's device-side
    pass on at most overlap_kernel_max_workgroups workgroups, whose waves then
    stride over the 1 KiB windows. With caps of 1, 3 and 96 workgroups, for
    narrow, half-window and wide rows in every layout, the loaded device pool
    matches the oracle, and the last pass launched no more workgroups than the
    cap."""
    for layout in LAYOUTS:
        g = Geometry(3, 2, R, 640, 512, 16, layout)
        bufs = device_buffers(g, seed=40 + layout)
        rng = np.random.default_rng(40 + layout)
        d = rng.permutation(g.S_dev)[:400].astype(np.int64)
        h = rng.permutation(g.S_host)[:400].astype(np.int64)
        pool = make_pool(g, bufs, path=kvt.PATH_STAGED,
                         flags=kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP, host_fill=None)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        c = pool.calibration()
        for cap in (1, 3, 96):
            print("staged capped R=%d layout=%d cap=%d" % (R, layout, cap), flush=True)
            c.overlap_kernel_max_workgroups = cap
            c.staged_chunk_bytes = 64 * 1024      # several chunks, ramped
            pool.set_calibration(c)
            run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
            assert pool.last_path(kvt.LOAD) == kvt.PATH_STAGED
            assert 1 <= pool.stats().last_workgroups[1] <= cap
            run_load_and_compare(g, pool, bufs, d[:123], h[:123], 1, 3, stream)
            assert 1 <= pool.stats().last_workgroups[1] <= cap
        pool.close()


def _hold_stream(torch, st, gate):
    """Enqueues on `st` a host function that returns once `gate` is set (or after
    10 s): work queued behind it stays in flight until then."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")     # the runtime torch has loaded
    fn_t = ctypes.CFUNCTYPE(None, ctypes.c_void_p)
    cb = fn_t(lambda _: gate.wait(10.0))
    hip.hipLaunchHostFunc.argtypes = [ctypes.c_void_p, fn_t, ctypes.c_void_p]
    assert hip.hipLaunchHostFunc(ctypes.c_void_p(st.cuda_stream), cb, None) == 0
    return cb                                  # keep the callback alive until the stream passes it


def test_duplex_caps_follow_the_other_direction(torch):
    """Without KV_F_DUPLEX the duplex grid caps apply while the other direction
    has a transfer in flight on another stream at submission: a backup issued
    while a load is held in flight gets 8 workgroups and a load issued while a
    backup is held gets 32; issued alone, each gets the full grid. Both
    directions' bytes match the oracle."""
    import threading
    g = Geometry(4, 2, 2048, 8192, 8192, 64, 0)
    bufs = device_buffers(g, seed=16)
    pool = make_pool(g, bufs, kvt.PATH_KERNEL, host_fill=None)
    c = pool.calibration()
    c.kernel_max_workgroups[0] = 0           # backups alone on a full grid
    pool.set_calibration(c)
    rng = np.random.default_rng(16)
    pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
    half = g.S_dev // 2
    d_load, h_load = np.arange(half, dtype=np.int64), rng.permutation(half).astype(np.int64)
    d_back = np.arange(half, g.S_dev, dtype=np.int64)
    h_back = (half + rng.permutation(half)).astype(np.int64)
    s_load, s_back = torch.cuda.Stream(), torch.cuda.Stream()
    full_backup = g.S_dev // 2 * g.L * g.C * g.R // (16 * 1024)
    full_load = g.S_dev // 2 * g.C * g.R // (16 * 1024)      # one layer per launch

    for first in ("load", "backup"):
        print("duplex caps, %s held in flight" % first, flush=True)
        dev_m = mirrors(bufs)
        host_m = pool.host_array().copy()
        assert oracle.backup(g, dev_m, host_m, d_back, h_back) == 0   # disjoint rows:
        assert oracle.load(g, dev_m, host_m, d_load, h_load) == 0     # order is irrelevant
        gate = threading.Event()
        torch.cuda.synchronize()
        if first == "load":
            cb = _hold_stream(torch, s_load, gate)
            pool.load(d_load, h_load, 0, g.L, s_load)
            pool.backup(d_back, h_back, 0, g.L, s_back)
            grids = tuple(pool.stats().last_workgroups)
            assert grids == (8, full_load), grids
        else:
            cb = _hold_stream(torch, s_back, gate)
            pool.backup(d_back, h_back, 0, g.L, s_back)
            pool.load(d_load, h_load, 0, g.L, s_load)
            grids = tuple(pool.stats().last_workgroups)
            assert grids == (full_backup, 32), grids
        gate.set()
        s_load.synchronize()
        s_back.synchronize()
        torch.cuda.synchronize()
        del cb
        assert np.array_equal(pool.host_array(), host_m)
        for k, b in enumerate(bufs):
            assert np.array_equal(b.cpu().numpy(), dev_m[k]), k
    # alone again: full grids
    pool.backup(d_back, h_back, 0, g.L, s_back)
    s_back.synchronize()
    pool.load(d_load, h_load, 0, g.L, s_load)
    s_load.synchronize()
    assert tuple(pool.stats().last_workgroups) == (full_backup, full_load)
    pool.close()


@pytest.mark.parametrize("path", PATHS)
def test_null_stream_round_trip(torch, path):
    """A NULL stream means the null stream: backup and load issued there (no
    stream argument) match the oracle on every path, and kv_load_layer on the
    null stream orders a consumer there after the layer."""
    L, C, R, S_dev, S_host, ps = GEOMS[0]
    for layout in LAYOUTS:
        g = Geometry(L, C, R, S_dev, S_host, ps, layout)
        bufs = device_buffers(g, seed=17 + layout)
        pool = make_pool(g, bufs, path)
        rng = np.random.default_rng(17 + layout)
        d, h = _request(rng, g, "random")
        print("null stream path=%d layout=%d" % (path, layout), flush=True)
        want = pool.host_array().copy()
        assert oracle.backup(g, mirrors(bufs), want, d, h) == 0
        torch.cuda.synchronize()
        pool.backup(d, h, 0, L)
        torch.cuda.synchronize()
        assert np.array_equal(pool.host_array(), want)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        dev_m = mirrors(bufs)
        assert oracle.load(g, dev_m, pool.host_array().copy(), d, h) == 0
        pool.load(d, h, 0, L)
        pool.load_layer(L - 1)
        t_idx = torch.from_numpy(d).cuda()
        last = bufs[(L - 1) * C].view(-1, g.R).index_select(0, t_idx).cpu().numpy()
        assert np.array_equal(last, dev_m[(L - 1) * C].reshape(-1, g.R)[d])
        torch.cuda.synchronize()
        for k, b in enumerate(bufs):
            assert np.array_equal(b.cpu().numpy(), dev_m[k]), k
        pool.close()


@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED))
def test_destroy_waits_for_work_in_flight(torch, path):
    """kv_pool_destroy right after enqueueing: it waits for the pool's transfers
    before freeing anything. A load's rows land in full; a writer's backup lands
    in the host pool a sharing pool keeps alive, and both match the oracle."""
    g = Geometry(4, 2, 2048, 16384, 16384, 64, 0)
    rng = np.random.default_rng(18)
    d = rng.permutation(g.S_dev)[:12288].astype(np.int64)
    h = rng.permutation(g.S_host)[:12288].astype(np.int64)
    s = torch.cuda.Stream()
    # load, then destroy at once
    bufs = device_buffers(g, seed=18)
    pool = make_pool(g, bufs, path, host_fill=None)
    pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
    dev_m = mirrors(bufs)
    assert oracle.load(g, dev_m, pool.host_array().copy(), d, h) == 0
    torch.cuda.synchronize()
    print("destroy during a load, path=%d" % path, flush=True)
    pool.load(d, h, 0, g.L, s)
    pool.close()
    torch.cuda.synchronize()
    for k, b in enumerate(bufs):
        assert np.array_equal(b.cpu().numpy(), dev_m[k]), k
    # backup by a writer destroyed at once; a sharing pool holds the host pool
    writer = make_pool(g, bufs, path)
    reader = kvt.KvPool(kv_geom(g), device_buffers(g, seed=19), share_with=writer)
    want = writer.host_array().copy()
    assert oracle.backup(g, mirrors(bufs), want, d, h) == 0
    torch.cuda.synchronize()
    print("destroy during a backup, path=%d" % path, flush=True)
    writer.backup(d, h, 0, g.L, s)
    writer.close()
    torch.cuda.synchronize()
    assert np.array_equal(reader.host_array(), want)
    reader.close()


def test_selector_models_capped_grids_per_workgroup(torch, stream):
    """AUTO prices a capped kernel by what its workgroups move: a backup of 512
    blocks on a 24-workgroup grid, at 10 GB/s per workgroup, loses to two
    copy-engine copies; on a full grid (512 workgroups) it wins. Bytes match
    the oracle on both paths. Unpaced: the per-workgroup terms are priced."""
    g = Geometry(2, 1, 4096, 1024, 1024, 8, 0)
    bufs = device_buffers(g, seed=20)
    pool = make_pool(g, bufs, kvt.PATH_AUTO)
    d, h = np.arange(1024, dtype=np.int64), np.arange(1024, dtype=np.int64)
    c = pool.calibration()
    assert c.kernel_wg_gbps[0] > 0 and c.kernel_wg_row_ns[0] >= 0
    c.kernel_launch_us[0], c.dma_copy_us[0] = 15.0, 10.0        # kernel 15 us, copies 2 x 10 us
    c.kernel_gbps[0] = c.dma_gbps[0] = 1e6                       # link terms negligible
    c.kernel_wg_gbps[0], c.kernel_wg_row_ns[0] = 10.0, 0.0      # 8 MiB / (24 x 10 GB/s) = 35 us
    c.kernel_max_workgroups[0] = 24
    c.kernel_pace_gbps[0] = 0.0
    pool.set_calibration(c)
    run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_DMA
    c.kernel_max_workgroups[0] = 0                                # 512 workgroups: 1.6 us
    pool.set_calibration(c)
    run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_KERNEL
    # the capped grid's slow start: 100 us over the first 16 MiB, of which the
    # 8 MiB call pays half; the per-workgroup rate itself is made negligible
    c.kernel_max_workgroups[0] = 24
    c.kernel_wg_gbps[0] = 1e6
    for start_us, want in ((0.0, kvt.PATH_KERNEL), (100.0, kvt.PATH_DMA)):
        c.kernel_wg_start_bytes[0], c.kernel_wg_start_us[0] = 16 * 2 ** 20, start_us
        pool.set_calibration(c)
        run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        assert pool.last_path(kvt.BACKUP) == want, start_us
    c.kernel_max_workgroups[0] = 0                                # not capped: no slow start
    pool.set_calibration(c)
    run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_KERNEL
    c.kernel_wg_start_us[0] = -1.0
    with pytest.raises(kvt.KvError):
        pool.set_calibration(c)
    c.kernel_wg_start_us[0] = 0.0
    c.kernel_wg_gbps[0] = 0.0
    with pytest.raises(kvt.KvError):
        pool.set_calibration(c)
    pool.close()


def test_overlap_flag_steers_selector(torch, stream):
    g = Geometry(2, 1, 64, 32, 32, 8, 0)
    bufs = device_buffers(g, seed=12)
    d, h = np.arange(8), np.arange(8)
    for flags, want in ((kvt.F_CHECK_UNIQUE, kvt.PATH_KERNEL),
                        (kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP, kvt.PATH_DMA)):
        pool = make_pool(g, bufs, kvt.PATH_AUTO, flags=flags)
        c = pool.calibration()
        # two 1-D copies at 10 us each against one launch at 15 us: the kernel wins
        # alone; charged overlap penalties of x1.65 vs x1.15 the copy
        # engines win
        c.kernel_launch_us[1], c.dma_copy_us[1] = 15.0, 10.0
        c.kernel_gbps[1] = c.dma_gbps[1] = 1e6
        c.overlap_kernel_penalty, c.overlap_dma_penalty = 0.65, 0.15
        pool.set_calibration(c)
        run_load_and_compare(g, pool, bufs, d, h, 0, 2, stream)
        assert pool.last_path(kvt.LOAD) == want
        # backups are never charged the overlap penalty
        c.kernel_launch_us[0], c.dma_copy_us[0] = 15.0, 10.0
        c.kernel_gbps[0] = c.dma_gbps[0] = 1e6
        pool.set_calibration(c)
        pool.backup(d, h, 0, 2, stream)
        stream.synchronize()
        assert pool.last_path(kvt.BACKUP) == kvt.PATH_KERNEL
        pool.close()


@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA))
def test_load_layer_groups_gate_consumer(torch, path):
    """Layers loaded in groups of three (one launch and one landed event per
    group): a consumer that waits with kv_load_layer(l) sees layer l complete,
    and the bytes equal the oracle's."""
    g = Geometry(8, 2, 512, 4096, 4096, 16, oracle.LAYER_FIRST)
    n = 4096
    bufs = device_buffers(g, seed=13, fill=0)
    pool = make_pool(g, bufs, path, host_fill=None)
    pool.host_array()[:] = np.random.default_rng(13).integers(0, 256, g.host_bytes(), np.uint8)
    c = pool.calibration()
    c.load_split_min_bytes = 10 * 1024 * 1024        # a layer is 4 MiB -> groups of 3
    pool.set_calibration(c)
    d = np.random.default_rng(14).permutation(g.S_dev)[:n]
    h = np.arange(n)
    mirrors = [np.zeros(g.S_dev * g.R, np.uint8) for _ in range(g.L * g.C)]
    assert oracle.load(g, mirrors, pool.host_array(), d, h) == 0
    s_load, s_comp = torch.cuda.Stream(), torch.cuda.Stream()
    t_idx = torch.from_numpy(d).cuda()
    torch.cuda.synchronize()
    before = pool.stats().kernel_launches[1]
    pool.load(d, h, 0, g.L, s_load)
    with torch.cuda.stream(s_comp):
        # made on the consumer's stream, so no other stream's fill can land on it late
        sums = torch.zeros(g.L * g.C, dtype=torch.int64, device="cuda:0")
        for l in range(g.L):
            pool.load_layer(l, s_comp)
            for cc in range(g.C):
                rows = bufs[l * g.C + cc].view(-1, g.R).index_select(0, t_idx)
                sums[l * g.C + cc] = rows.to(torch.int64).sum()
    s_comp.synchronize()
    s_load.synchronize()
    for k in range(g.L * g.C):
        want = mirrors[k].reshape(g.S_dev, g.R)[d].astype(np.int64).sum()
        assert int(sums[k]) == int(want), k
        assert np.array_equal(bufs[k].cpu().numpy(), mirrors[k]), k
    if path == kvt.PATH_KERNEL:
        assert pool.stats().kernel_launches[1] - before == 3
    pool.close()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_staged_small_chunks_match_oracle(torch, stream, layout):
    """A staging buffer of a few rows: many chunks, extents split across chunk
    boundaries, layer groups on loads."""
    L, C, R, S_dev, S_host, ps = GEOMS[0]
    g = Geometry(L, C, R, S_dev, S_host, ps, layout)
    bufs = device_buffers(g, seed=15)
    rng = np.random.default_rng(15 + layout)
    pool = make_pool(g, bufs, kvt.PATH_STAGED)
    for chunk_rows, split_rows in ((3, 10 ** 9), (37, 50), (1000, 1)):
        c = pool.calibration()
        c.staged_chunk_bytes = chunk_rows * R
        c.load_split_min_bytes = split_rows * R
        pool.set_calibration(c)
        for kind in ("random", "contiguous", "pages"):
            d, h = _request(rng, g, kind)
            print("staged layout=%d chunk=%d kind=%s" % (layout, chunk_rows, kind), flush=True)
            run_backup_and_compare(g, pool, bufs, d, h, 0, L, stream)
            pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            run_load_and_compare(g, pool, bufs, d, h, 1, L, stream)
            assert pool.last_path(kvt.LOAD) == kvt.PATH_STAGED
    pool.close()


def _ramp_chunks(walk_rows, chunk_rows, ramp):
    """Chunk count of a staged unit: full chunks, or chunks growing 8x from
    1/64 of a chunk where the ramp applies (same count at either end)."""
    if not ramp:
        return -(-walk_rows // chunk_rows)
    n, r, ln = 0, 0, max(1, chunk_rows // 64)
    while r < walk_rows:
        r += min(ln, walk_rows - r)
        n += 1
        ln = min(chunk_rows, ln * 8)
    return n


@pytest.mark.parametrize("layout", LAYOUTS)
def test_staged_ramp_chunks(torch, stream, layout):
    """The staged path's chunk ramp: a backup's first chunks and a load's last
    ones grow 8x from 1/64 of a staging half when the half is at least 1/16
    of staged_chunk_bytes, else every chunk fills the half. One launch per
    chunk (kv_get_stats); bytes match the oracle."""
    g = Geometry(2, 1, 64, 2048, 2048, 8, layout)
    bufs = device_buffers(g, seed=16)
    rng = np.random.default_rng(16 + layout)
    pool = make_pool(g, bufs, kvt.PATH_STAGED)
    n = 500
    d = rng.permutation(g.S_dev)[:n].astype(np.int64)
    h = np.arange(100, 100 + n, dtype=np.int64)
    walk = n * g.L * g.C
    # (chunk rows, load group rows, expected backup / load launches)
    cases = [(64, 10 ** 9, _ramp_chunks(walk, 64, True), _ramp_chunks(walk, 64, True)),
             (100000, 10 ** 9, 1, 1)]
    if layout == oracle.LAYER_FIRST:   # per-layer load groups: only the last one ramps
        cases.append((64, 1, _ramp_chunks(walk, 64, True),
                      _ramp_chunks(n, 64, False) + _ramp_chunks(n, 64, True)))
    for chunk_rows, split_rows, want_b, want_l in cases:
        c = pool.calibration()
        c.staged_chunk_bytes = chunk_rows * g.R
        c.load_split_min_bytes = split_rows * g.R
        pool.set_calibration(c)
        print("staged ramp layout=%d chunk=%d split=%d" % (layout, chunk_rows, split_rows),
              flush=True)
        before = pool.stats().kernel_launches[:]
        run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        after = pool.stats().kernel_launches[:]
        assert (after[0] - before[0], after[1] - before[1]) == (want_b, want_l)
    pool.close()


# ---- streams with a hardware queue of their own ---------------------------------------

@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED))
def test_library_streams_round_trip(torch, path):
    """Backup and load issued on kv_stream_create streams, at the same time,
    match the oracle; bad arguments are rejected."""
    shape = workloads.tiny()
    g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                 shape.host_slots, shape.page_size, oracle.LAYER_FIRST)
    assert kvt.kv_stream_create(-1)[0] == kvt.EINVAL
    assert kvt.kv_stream_create(torch.cuda.device_count())[0] == kvt.EINVAL
    assert kvt.kv_stream_destroy(None) == kvt.OK
    dev_idx, host_idx, reload_idx = workloads.tiny_indices(shape)
    src = device_buffers(g, seed=11)
    pool = make_pool(g, src, path)
    s_back, s_load = kvt.Stream(), kvt.Stream()
    print("library streams path=%d" % path, flush=True)
    run_backup_and_compare(g, pool, src, dev_idx, host_idx, 0, g.L, s_back)
    # load into a second pool on one stream while the first backs up again on the other
    fresh = device_buffers(g, seed=12, fill=SENTINEL)
    pool2 = make_pool(g, fresh, path, host_fill=None)
    pool2.host_array()[:] = pool.host_array()
    want_dev = mirrors(fresh)
    assert oracle.load(g, want_dev, pool2.host_array().copy(), reload_idx, host_idx) == 0
    want_host = pool.host_array().copy()
    pool2.load(reload_idx, host_idx, 0, g.L, s_load)
    pool.backup(dev_idx, host_idx, 0, g.L, s_back)
    s_load.synchronize()
    s_back.synchronize()
    assert np.array_equal(pool.host_array(), want_host)
    for k, b in enumerate(fresh):
        assert np.array_equal(b.cpu().numpy(), want_dev[k]), k
    s_back.close()
    s_load.close()
    pool.close()
    pool2.close()


def test_staged_margin_steers_selector(torch, stream):
    """AUTO takes the staged path only when its modelled time beats the best
    direct path by staged_min_gain; bytes match the oracle either way."""
    g = Geometry(2, 1, 64, 256, 256, 8, oracle.LAYER_FIRST)
    bufs = device_buffers(g, seed=14)
    rng = np.random.default_rng(14)
    d = rng.permutation(g.S_dev)[:64].astype(np.int64)   # 64 single-slot device runs
    h = np.arange(64, dtype=np.int64)                     # one host run per layer
    pool = make_pool(g, bufs, kvt.PATH_AUTO, flags=kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX)
    c = pool.calibration()
    # kernel: 10 us x (1 + 100) = 1010 us; copy engines: 128 copies x 100 us;
    # staged: 2 extents x 100 us + 10 us + 7 us + ~0 = ~217 us
    c.kernel_launch_us[:] = [10.0, 10.0]
    c.kernel_group_us[:] = [7.0, 7.0]
    c.dma_copy_us[:] = [100.0, 100.0]
    c.kernel_gbps[:] = [1e6, 1e6]
    c.dma_gbps[:] = [1e6, 1e6]
    c.staged_gather_gbps = 1e6
    c.duplex_kernel_penalty[:] = [100.0, 100.0]
    for gain, want in ((0.9, kvt.PATH_KERNEL), (0.5, kvt.PATH_STAGED)):
        c.staged_min_gain = gain
        pool.set_calibration(c)
        print("staged margin gain=%.1f" % gain, flush=True)
        run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        assert pool.last_path(kvt.BACKUP) == want
        pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        assert pool.last_path(kvt.LOAD) == want
    c.staged_min_gain = 1.0
    with pytest.raises(kvt.KvError):
        pool.set_calibration(c)
    pool.close()


def test_overlapped_page_major_loads_skip_staged(torch, stream):
    """With KV_F_LOAD_OVERLAP, AUTO leaves the staged path out of page_first /
    page_first_direct loads (one unit: every layer would land at the end), but
    keeps it for layer_first loads, whose layer groups land one by one. The
    calibration makes the staged path the cheapest in every case; bytes match
    the oracle."""
    rng = np.random.default_rng(21)
    d = rng.permutation(256)[:64].astype(np.int64)   # 64 single-slot device runs
    h = np.arange(64, dtype=np.int64)                 # one host run
    for layout in LAYOUTS:
        g = Geometry(2, 1, 64, 256, 256, 8, layout)
        bufs = device_buffers(g, seed=21)
        for flags in (kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX,
                      kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX | kvt.F_LOAD_OVERLAP):
            pool = make_pool(g, bufs, kvt.PATH_AUTO, flags=flags)
            c = pool.calibration()
            # kernel: 10 us x (1 + 100) (x 1.65 overlapped); copy engines: one
            # copy per device run at 100 us; staged: a copy per host extent
            c.kernel_launch_us[:] = [10.0, 10.0]
            c.kernel_group_us[:] = [7.0, 7.0]
            c.dma_copy_us[:] = [100.0, 100.0]
            c.kernel_gbps[:] = [1e6, 1e6]
            c.dma_gbps[:] = [1e6, 1e6]
            c.staged_gather_gbps = 1e6
            c.duplex_kernel_penalty[:] = [100.0, 100.0]
            pool.set_calibration(c)
            pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            print("overlap staged layout=%d flags=%d" % (layout, flags), flush=True)
            run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
            skip = (flags & kvt.F_LOAD_OVERLAP) and layout != oracle.LAYER_FIRST
            assert (pool.last_path(kvt.LOAD) == kvt.PATH_STAGED) != skip, (layout, flags)
            pool.close()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_auto_takes_the_path_the_model_names(torch, stream, layout):
    """kv_model_path (host only) and a pool's AUTO choice agree on the same
    request and calibration, for small and fragmented requests in both
    directions; the bytes match the oracle."""
    g = Geometry(6, 2, 1024, 512, 512, 16, layout)
    bufs = device_buffers(g, seed=22)
    rng = np.random.default_rng(22 + layout)
    geom = kvt.geometry(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout)
    pool = make_pool(g, bufs, kvt.PATH_AUTO)
    calib = pool.calibration()
    for kind in ("contiguous", "random", "pages"):
        d, h = _request(rng, g, kind)
        for dirn in (kvt.BACKUP, kvt.LOAD):
            want, _ = kvt.kv_model_path(geom, calib, dirn, d, h, 0, g.L)
            assert want in (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED)
            print("model vs auto layout=%d kind=%s dir=%d" % (layout, kind, dirn), flush=True)
            if dirn == kvt.BACKUP:
                run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
            else:
                pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
                run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
            assert pool.last_path(dirn) == want, (kind, dirn)
    pool.close()


# ---- host pages handed out by the free list under churn --------------------------------

@pytest.mark.parametrize("policy", (kvt.FREE_FIFO, kvt.FREE_LIFO), ids=["fifo", "lifo"])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_churn_through_free_list(torch, stream, policy, layout):
    """Write-backs into pages from the library's free list while old requests are
    evicted (LIFO hands out fragmented runs of recently freed pages), then a load
    of every cached request; the oracle gets its pages from the oracle's free list."""
    from oracle import slots as oracle_slots
    g = Geometry(3, 2, 272, 640, 640, 16, layout)
    pages_total, cap = g.S_host // g.ps, 16
    bufs = device_buffers(g, seed=31)
    rng = np.random.default_rng(7 + policy)
    lib_alloc = kvt.HostPages(pages_total, policy)
    ref_alloc = oracle_slots.FreeList(pages_total, policy)
    for path in (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED, kvt.PATH_AUTO):
        pool = make_pool(g, bufs, path)
        live, live_pages = [], 0
        for r in range(24):
            npg = int(rng.integers(1, 9))
            while live_pages + npg > cap:
                old = live.pop(0)
                lib_alloc.free(old)
                assert ref_alloc.release(old.tolist()) == oracle_slots.OK
                live_pages -= old.size
            pages = lib_alloc.alloc(npg)
            rc, ref_pages = ref_alloc.alloc(npg)
            assert rc == oracle_slots.OK and pages.tolist() == ref_pages
            live.append(pages)
            live_pages += npg
            first = int(rng.integers(0, g.S_dev // g.ps - npg + 1))
            d = workloads.page_indices(np.arange(first, first + npg), g.ps)
            h = workloads.page_indices(np.asarray(ref_pages), g.ps)
            print("churn policy=%d layout=%d path=%d request=%d pages=%s" %
                  (policy, layout, path, r, ref_pages), flush=True)
            run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        h_all = workloads.page_indices(np.concatenate(live), g.ps)
        d_all = np.arange(h_all.size, dtype=np.int64)
        fresh = device_buffers(g, seed=32, fill=SENTINEL)
        pool2 = make_pool(g, fresh, path, host_fill=None)
        pool2.host_array()[:] = pool.host_array()
        run_load_and_compare(g, pool2, fresh, d_all, h_all, 0, g.L, stream)
        pool2.close()
        pool.close()
        for old in live:
            lib_alloc.free(old)
            assert ref_alloc.release(old.tolist()) == oracle_slots.OK
    lib_alloc.close()


# ---- one host pool shared by a tensor-parallel group -----------------------------------

def _random_request(rng, g, n, S_dev=None):
    S_dev = g.S_dev if S_dev is None else S_dev
    return (rng.choice(S_dev, n, replace=False).astype(np.int64),
            rng.choice(g.S_host, n, replace=False).astype(np.int64))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED, kvt.PATH_AUTO))
def test_shared_host_pool_group(torch, stream, layout, path):
    """The writer backs up; the sharing pools' backups move nothing; every pool
    loads the writer's bytes into its own device buffers at its own slots."""
    g = Geometry(3, 2, 272, 600, 512, 16, layout)
    rng = np.random.default_rng(40 + 10 * layout + path)
    src = device_buffers(g, seed=41)
    writer = make_pool(g, src, path)
    g2 = Geometry(3, 2, 272, 900, 512, 16, layout)         # a rank with a larger device pool
    readers = []
    for gr, seed in ((g, 42), (g2, 43)):
        bufs = device_buffers(gr, seed=seed, fill=SENTINEL)
        pr = kvt.KvPool(kv_geom(gr), bufs, share_with=writer)
        pr.set_path(path)
        readers.append((gr, pr, bufs))
    assert readers[0][1].host_array().ctypes.data == writer.host_array().ctypes.data
    d, h = _random_request(rng, g, 300)
    print("shared layout=%d path=%d" % (layout, path), flush=True)
    run_backup_and_compare(g, writer, src, d, h, 0, g.L, stream)
    image = writer.host_array().copy()
    for gr, pr, bufs in readers:
        d_r = rng.choice(gr.S_dev, h.size, replace=False).astype(np.int64)
        pr.backup(d_r, h, 0, g.L, stream)
        stream.synchronize()
        assert pr.last_path(kvt.BACKUP) == kvt.PATH_SHARED
        assert pr.stats().bytes[0] == 0 and pr.stats().calls[0] == 1
        assert np.array_equal(writer.host_array(), image)
        run_load_and_compare(gr, pr, bufs, d_r, h, 0, g.L, stream)
        for k in range(g.L * g.C):   # the rank's rows are the writer's source rows
            a = src[k].view(g.S_dev, g.R)[torch.from_numpy(d).cuda()]
            b = bufs[k].view(gr.S_dev, gr.R)[torch.from_numpy(d_r).cuda()]
            assert torch.equal(a, b)
    for _, pr, _ in readers:
        pr.close()
    writer.close()


def test_shared_backup_waits_for_the_writer(torch):
    """A sharing pool's backup and load on another stream, issued right after
    the writer's backup with no host synchronisation, see the written bytes."""
    g = Geometry(8, 2, 2048, 8192, 8192, 64, kvt.LAYER_FIRST)   # 256 MiB per direction
    rng = np.random.default_rng(44)
    src = device_buffers(g, seed=45)
    writer = make_pool(g, src, kvt.PATH_DMA)
    bufs = device_buffers(g, seed=46, fill=SENTINEL)
    reader = kvt.KvPool(kv_geom(g), bufs, share_with=writer)
    reader.set_path(kvt.PATH_KERNEL)
    s_w, s_r = torch.cuda.Stream(), torch.cuda.Stream()
    pages = rng.permutation(g.S_dev // g.ps)
    d = workloads.page_indices(pages, g.ps)
    h = np.arange(g.S_host, dtype=np.int64)
    d_r = workloads.page_indices(rng.permutation(g.S_dev // g.ps), g.ps)
    for rep in range(3):
        writer.host_array()[:] = SENTINEL
        for b in bufs:
            b.fill_(SENTINEL)
        torch.cuda.synchronize()
        print("shared gating rep=%d" % rep, flush=True)
        writer.backup(d, h, 0, g.L, s_w)
        reader.backup(d_r, h, 0, g.L, s_r)
        reader.load(d_r, h, 0, g.L, s_r)
        s_r.synchronize()
        for k in range(g.L * g.C):
            a = src[k].view(g.S_dev, g.R)[torch.from_numpy(d).cuda()]
            b = bufs[k].view(g.S_dev, g.R)[torch.from_numpy(d_r).cuda()]
            assert torch.equal(a, b), (rep, k)
        s_w.synchronize()
    reader.close()
    writer.close()


def test_shared_check_and_errors(torch, stream):
    g = Geometry(2, 1, 64, 128, 128, 8, kvt.PAGE_FIRST_DIRECT)
    rng = np.random.default_rng(47)
    src = device_buffers(g, seed=48)
    writer = make_pool(g, src, kvt.PATH_KERNEL, flags=kvt.F_CHECK_UNIQUE | kvt.F_SHARE_CHECK)
    bufs = device_buffers(g, seed=49, fill=SENTINEL)
    reader = kvt.KvPool(kv_geom(g), bufs, share_with=writer)
    lib = kvt.library()
    d, h = _random_request(rng, g, 40)
    # before the writer has backed up anything
    assert kvt.kv_backup(reader.handle, d, h, 0, g.L, stream) == kvt.EINVAL
    writer.backup(d, h, 0, g.L, stream)
    assert kvt.kv_backup(reader.handle, d[::-1], h, 0, g.L, stream) == kvt.OK  # own device slots
    assert kvt.kv_backup(reader.handle, d, h[::-1], 0, g.L, stream) == kvt.EINVAL
    assert "host allocation differs" in kvt.kv_last_error()
    assert kvt.kv_backup(reader.handle, d, h, 1, g.L, stream) == kvt.EINVAL
    # validation comes first, with the codes a backup gives
    bad = h.copy()
    bad[3] = g.S_host
    assert kvt.kv_backup(reader.handle, d, bad, 0, g.L, stream) == kvt.ERANGE
    dup = h.copy()
    dup[3] = dup[4]
    assert kvt.kv_backup(reader.handle, d, dup, 0, g.L, stream) == kvt.EDUP
    assert kvt.kv_backup(reader.handle, d, h, 0, 0, stream) == kvt.OK        # empty: no check
    # geometry must match the group's (all but device_slots)
    for other in (Geometry(2, 1, 80, 128, 128, 8, g.layout), Geometry(2, 1, 64, 128, 256, 8, g.layout),
                  Geometry(2, 1, 64, 128, 128, 8, kvt.LAYER_FIRST)):
        ob = device_buffers(other, seed=1, fill=0)
        rc, hnd = kvt.kv_pool_create_shared(kv_geom(other), [b.data_ptr() for b in ob],
                                            writer.handle)
        assert rc == kvt.EINVAL and not hnd
    assert kvt.kv_pool_create_shared(kv_geom(g), [b.data_ptr() for b in bufs], None)[0] == kvt.EINVAL
    # the host pool outlives the writer
    stream.synchronize()
    image = writer.host_array().copy()
    writer.close()
    assert np.array_equal(reader.host_array(), image)
    run_load_and_compare(g, reader, bufs, d, h, 0, g.L, stream)
    reader.close()
    assert lib.kv_pool_destroy(None) == kvt.OK


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("path", PATHS)
def test_back_to_back_on_one_stream(torch, stream, layout, path):
    """A backup and a load of the same host slots chained on one stream with no
    host synchronisation between them (the load must read what the backup
    wrote), three times over with different device slots."""
    g = Geometry(4, 2, 1152, 2048, 1024, 64, layout)
    rng = np.random.default_rng(60 + 10 * layout + path)
    src = device_buffers(g, seed=61)
    pool = make_pool(g, src, path)
    dst = device_buffers(g, seed=62, fill=SENTINEL)
    pool2 = kvt.KvPool(kv_geom(g), dst, share_with=pool)   # loads into other buffers
    pool2.set_path(path)
    h = rng.permutation(g.S_host).astype(np.int64)
    for rep in range(3):
        d_src = rng.choice(g.S_dev, g.S_host, replace=False).astype(np.int64)
        d_dst = rng.choice(g.S_dev, g.S_host, replace=False).astype(np.int64)
        print("back-to-back layout=%d path=%d rep=%d" % (layout, path, rep), flush=True)
        pool.backup(d_src, h, 0, g.L, stream)
        pool2.load(d_dst, h, 0, g.L, stream)
        stream.synchronize()
        for k in range(g.L * g.C):
            a = src[k].view(g.S_dev, g.R)[torch.from_numpy(d_src).cuda()]
            b = dst[k].view(g.S_dev, g.R)[torch.from_numpy(d_dst).cuda()]
            assert torch.equal(a, b), (rep, k)
    pool2.close()
    pool.close()


def test_request_row_limit(torch, stream):
    """A call moves fewer than 2^31 rows (n x layers x components): a request of
    exactly 2^31 rows is refused in both directions before anything is enqueued.
    2048 (layer, component) buffers alias one 16 MiB device allocation and every
    request position names host slot 0 (no uniqueness check), so the pools stay
    small; only the refusal is exercised, no transfer runs."""
    L, C, R, S_dev = 1024, 2, 16, 1 << 20
    one = torch.zeros(S_dev * R, dtype=torch.uint8, device="cuda:0")
    kg = kvt.geometry(L, C, R, S_dev, 1, 1, kvt.LAYER_FIRST)
    rc, h = kvt.kv_pool_create(kg, [one.data_ptr()] * (L * C), flags=0)
    assert rc == kvt.OK, kvt.kv_last_error()
    n = (1 << 31) // (L * C)                       # exactly 2^31 rows over all layers
    d = np.arange(n, dtype=np.int64)
    hz = np.zeros(n, dtype=np.int64)
    for direction in (kvt.kv_backup, kvt.kv_load):
        assert direction(h, d, hz, 0, L, stream) == kvt.EINVAL
        assert "2^31" in kvt.kv_last_error()
    assert kvt.kv_get_stats(h)[1].calls[0] == 0 and kvt.kv_get_stats(h)[1].calls[1] == 0
    stream.synchronize()
    assert int(one.sum()) == 0
    assert kvt.kv_pool_destroy(h) == kvt.OK


def _fuzz_case(seed):
    """A seeded random geometry, request, layer range, layout and path."""
    rng = np.random.default_rng([7001, seed])
    L = int(rng.integers(1, 7))
    C = int(rng.integers(1, 3))
    R = 16 * int(rng.choice([1, 2, 3, 5, 8, 17, 64, 72, 128, 257]))
    ps = int(rng.choice([1, 2, 4, 16, 64]))
    S_host = ps * int(rng.integers(1, max(2, 1500 // ps)))
    S_dev = int(rng.integers(1, 1600))
    layout = int(rng.integers(0, 3))
    path = int(rng.choice(PATHS))
    n_max = min(S_dev, S_host)
    kind = rng.choice(["random", "contiguous", "pages", "tiny"])
    if kind == "tiny" or n_max < 2:
        n = int(rng.integers(0, min(3, n_max) + 1))
    else:
        n = int(rng.integers(1, n_max + 1))
    if kind == "contiguous":
        d0 = int(rng.integers(0, S_dev - n + 1))
        h0 = int(rng.integers(0, S_host - n + 1))
        d, h = np.arange(d0, d0 + n), np.arange(h0, h0 + n)
    elif kind == "pages" and S_host // ps >= 1 and S_dev >= ps:
        npg = int(rng.integers(1, min(S_dev // ps, S_host // ps) + 1))
        dp = rng.permutation(S_dev // ps)[:npg]
        hp = rng.permutation(S_host // ps)[:npg]
        d, h = workloads.page_indices(dp, ps), workloads.page_indices(hp, ps)
        cut = int(rng.integers(1, d.size + 1))       # a ragged last page
        d, h = d[:cut], h[:cut]
    else:
        d = rng.choice(S_dev, n, replace=False)
        h = rng.choice(S_host, n, replace=False)
    l0 = int(rng.integers(0, L + 1))
    l1 = int(rng.integers(l0, L + 1))
    if rng.random() < 0.5:
        l0, l1 = 0, L
    return (Geometry(L, C, R, S_dev, S_host, ps, layout), path, d.astype(np.int64),
            h.astype(np.int64), l0, l1)


@pytest.mark.parametrize("block", range(6))
def test_random_geometry_sweep(torch, stream, block):
    """100 seeded random cases per block: every layout and path, row sizes from 16
    bytes to 4 KiB, ragged page tails, partial layer ranges, empty requests."""
    for seed in range(100 * block, 100 * (block + 1)):
        g, path, d, h, l0, l1 = _fuzz_case(seed)
        print("sweep seed=%d L=%d C=%d R=%d S_dev=%d S_host=%d ps=%d layout=%d path=%d n=%d "
              "layers=[%d,%d)" % (seed, g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout, path,
                                  d.size, l0, l1), flush=True)
        bufs = device_buffers(g, seed=seed)
        pool = make_pool(g, bufs, path)
        run_backup_and_compare(g, pool, bufs, d, h, l0, l1, stream)
        pool.host_array()[:] = np.random.default_rng(seed).integers(
            0, 256, size=g.host_bytes(), dtype=np.uint8)
        run_load_and_compare(g, pool, bufs, d, h, l0, l1, stream)
        pool.close()


@pytest.mark.parametrize("zero_copy", (False, True), ids=["copied", "zero_copy"])
@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS, kvt.PATH_STAGED))
def test_index_pairs_copied_or_read_in_place(torch, stream, zero_copy, path):
    """The kernels take the request's index pairs either from a device copy or
    straight from the mapped pinned staging buffer (index_zero_copy_max_bytes);
    both give the oracle's bytes, for requests far above and below the default
    threshold, in every layout."""
    for layout in LAYOUTS:
        g = Geometry(3, 2, 272, 700, 640, 16, layout)
        bufs = device_buffers(g, seed=70 + layout)
        pool = make_pool(g, bufs, path)
        c = pool.calibration()
        c.index_zero_copy_max_bytes[:] = [1e18, 1e18] if zero_copy else [0.0, 0.0]
        pool.set_calibration(c)
        rng = np.random.default_rng(71 + layout)
        for n in (1, 5, 127, 600):
            d = rng.choice(g.S_dev, n, replace=False).astype(np.int64)
            h = rng.choice(g.S_host, n, replace=False).astype(np.int64)
            print("index pairs zero_copy=%d path=%d layout=%d n=%d" % (zero_copy, path, layout, n),
                  flush=True)
            run_backup_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
            pool.host_array()[:] = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            run_load_and_compare(g, pool, bufs, d, h, 0, g.L, stream)
        pool.close()


# ---- brute force: every permutation of tiny requests, oracle == NumPy == GPU ---------

@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("path", PATHS)
def test_brute_force_tiny_pools_on_gpu(torch, stream, layout, path):
    """Pools of L, C in {1, 2}, R in {16, 32} bytes, page size 1, 2 or 4 over 4 host
    slots (5 device slots): every ordered choice of 1-4 host slots is backed up from
    seeded device slots and loaded back into other seeded device slots. The C
    oracle and the NumPy cross-derivation agree on each result, and the library
    matches them byte for byte, the rest of both pools included."""
    S_host, S_dev = 4, 5
    cases = 0
    for L, C, R, ps in itertools.product((1, 2), (1, 2), (16, 32), (1, 2, 4)):
        g = Geometry(L, C, R, S_dev, S_host, ps, layout)
        rng = np.random.default_rng([8100, L, C, R, ps, layout, path])
        bufs = device_buffers(g, seed=int(rng.integers(1 << 30)))
        pool = make_pool(g, bufs, path)
        print("brute layout=%d path=%d L=%d C=%d R=%d ps=%d" % (layout, path, L, C, R, ps),
              flush=True)
        for n in (1, 2, 3, 4):
            for hs in itertools.permutations(range(S_host), n):
                h = np.asarray(hs, dtype=np.int64)
                d = rng.choice(S_dev, n, replace=False).astype(np.int64)
                # backup: oracle and NumPy from the same mirrors, then the library
                dev_m = mirrors(bufs)
                want = pool.host_array().copy()
                want_np = want.copy()
                assert oracle.backup(g, dev_m, want, d, h) == 0
                np_ref.backup(np.stack(dev_m).reshape(L, C, S_dev, R), want_np, layout, L, C,
                              S_host, ps, R, d, h)
                assert np.array_equal(want, want_np)
                pool.backup(d, h, 0, L, stream)
                stream.synchronize()
                assert np.array_equal(pool.host_array(), want), (L, C, R, ps, hs)
                # load into another seeded choice of device slots
                d2 = rng.choice(S_dev, n, replace=False).astype(np.int64)
                host = pool.host_array().copy()
                dev_m = mirrors(bufs)
                dev_np = np.stack(dev_m).reshape(L, C, S_dev, R).copy()
                assert oracle.load(g, dev_m, host, d2, h) == 0
                np_ref.load(dev_np, host, layout, L, C, S_host, ps, R, d2, h)
                pool.load(d2, h, 0, L, stream)
                stream.synchronize()
                for k, b in enumerate(bufs):
                    assert np.array_equal(dev_m[k], dev_np.reshape(L * C, -1)[k])
                    assert np.array_equal(b.cpu().numpy(), dev_m[k]), (L, C, R, ps, hs, k)
                cases += 1
        pool.close()
    assert cases == 24 * 64
