"""kv_transfer_noalloc, the entry point that allocates nothing, against the
entry points it varies (kv_backup / kv_load on the zero-copy kernel path),
through the C ABI: two calls in a row, the second with a smaller request, in
every layout and both directions; the results must be byte-identical to the
existing entry points' on identical pools (and, for the write-back, to the
oracle's host image)."""
import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
import oracle
from oracle import Geometry

from gpu_util import SENTINEL, device_buffers, kv_geom, mirrors, torch_mod

pytestmark = pytest.mark.gpu

MAX_POSITIONS = 1 << 18


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _requests(g, seed):
    """Two requests of one pool, the second smaller, disjoint destinations each."""
    rng = np.random.default_rng(seed)
    out = []
    for n in (g.S_host * 3 // 4 + 5, g.S_host // 5 + 3):
        d = rng.choice(g.S_dev, n, replace=False).astype(np.int64)
        h = rng.choice(g.S_host, n, replace=False).astype(np.int64)
        out.append((d, h))
    return out


@pytest.mark.parametrize("layout", (oracle.LAYER_FIRST, oracle.PAGE_FIRST,
                                    oracle.PAGE_FIRST_DIRECT))
@pytest.mark.parametrize("direction", (kvt.BACKUP, kvt.LOAD))
def test_noalloc_matches_the_kernel_path(torch, layout, direction):
    g = Geometry(5, 2, 272, 1500, 1024, 16, layout)
    print("noalloc layout=%d direction=%d" % (layout, direction), flush=True)
    bufs_a = device_buffers(g, seed=200 + layout)
    bufs_b = [b.clone() for b in bufs_a]
    pa = kvt.KvPool(kv_geom(g), bufs_a)          # existing entry points, kernel path
    pb = kvt.KvPool(kv_geom(g), bufs_b)          # kv_transfer_noalloc
    pa.set_path(kvt.PATH_KERNEL)
    rng = np.random.default_rng(300 + layout)
    init = rng.integers(0, 256, pa.host_array().size, dtype=np.uint8)
    pa.host_array()[:] = init
    pb.host_array()[:] = init
    want_host = init.copy()
    dev_m = mirrors(bufs_a)
    s = torch.cuda.Stream()
    for k, (d, h) in enumerate(_requests(g, 400 + layout + 10 * direction)):
        l0, l1 = (0, g.L) if k == 0 else (1, g.L - 1)
        if direction == kvt.BACKUP:
            pa.backup(d, h, l0, l1, s)
            assert oracle.backup(g, dev_m, want_host, d, h, l0, l1) == 0
        else:
            pa.load(d, h, l0, l1, s)
            assert oracle.load(g, dev_m, want_host, d, h, l0, l1) == 0
        rc = kvt.kv_transfer_noalloc(pb.handle, direction, d, h, l0, l1, s)
        assert rc == kvt.OK, kvt.kv_last_error()
        s.synchronize()
        assert pb.last_path(direction) == kvt.PATH_KERNEL
        assert np.array_equal(pb.host_array(), pa.host_array()), k
        assert np.array_equal(pb.host_array(), want_host), k
        for j, (x, y) in enumerate(zip(bufs_a, bufs_b)):
            assert torch.equal(x, y), (k, j)
            assert np.array_equal(y.cpu().numpy(), dev_m[j]), (k, j)
    pa.close()
    pb.close()


def test_noalloc_loads_land_per_layer(torch):
    """kv_load_layer gates a consumer after a no-allocation load as after kv_load."""
    L, R, n = 6, 1024, 8192
    g = Geometry(L, 1, R, 2 * n, n, 64, oracle.LAYER_FIRST)
    bufs = device_buffers(g, seed=9, fill=0)
    pool = kvt.KvPool(kv_geom(g), bufs)
    host = pool.host_array()
    host[:] = np.random.default_rng(10).integers(0, 256, host.size, dtype=np.uint8)
    c = pool.calibration()
    c.load_split_min_bytes = 1.0          # one group, one landed event per layer
    pool.set_calibration(c)
    s_load, s_comp = torch.cuda.Stream(), torch.cuda.Stream()
    dev_idx, host_idx = np.arange(n, 2 * n), np.arange(n)
    want = [int(host[l * n * R:(l + 1) * n * R].astype(np.int64).sum()) for l in range(L)]
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, dev_idx, host_idx, 0, L, s_load) == 0
    with torch.cuda.stream(s_comp):
        sums = torch.zeros(L, dtype=torch.int64, device="cuda:0")
        for l in range(L):
            pool.load_layer(l, s_comp)
            sums[l] = bufs[l].view(-1, R)[n:].to(torch.int64).sum()
    s_comp.synchronize()
    s_load.synchronize()
    assert [int(x) for x in sums.cpu()] == want
    pool.close()


def test_noalloc_refuses_oversized_and_bad_requests(torch):
    g = Geometry(1, 1, 16, MAX_POSITIONS + 8, MAX_POSITIONS + 16, 16, oracle.LAYER_FIRST)
    bufs = device_buffers(g, seed=11, fill=7)
    pool = kvt.KvPool(kv_geom(g), bufs)
    pool.host_array()[:] = SENTINEL
    s = torch.cuda.Stream()
    big = np.arange(MAX_POSITIONS + 1, dtype=np.int64)
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.BACKUP, big, big, 0, 1, s) == kvt.EINVAL
    assert "262144" in kvt.kv_last_error()
    s.synchronize()
    assert np.all(pool.host_array() == SENTINEL)           # nothing was enqueued
    top = np.arange(MAX_POSITIONS, dtype=np.int64)         # the largest request is taken
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.BACKUP, top, top, 0, 1, s) == kvt.OK
    s.synchronize()
    assert np.all(pool.host_array()[:MAX_POSITIONS * 16] == 7)
    assert np.all(pool.host_array()[MAX_POSITIONS * 16:] == SENTINEL)
    assert kvt.kv_transfer_noalloc(pool.handle, 2, top[:4], top[:4], 0, 1, s) == kvt.EINVAL
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, [3, 3], [1, 2], 0, 1, s) == kvt.EDUP
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, [3], [g.S_host], 0, 1, s) == kvt.ERANGE
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, [3], [2], 0, 2, s) == kvt.EINVAL
    assert kvt.kv_transfer_noalloc(None, kvt.LOAD, [3], [2], 0, 1, s) == kvt.EINVAL
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, [], [], 0, 1, s) == kvt.OK
    pool.close()


def test_noalloc_uniqueness_table_bound(torch):
    """A pool flagged KV_F_CHECK_UNIQUE sizes its uniqueness tables at creation
    for up to 2^24 destination slots. Past that, a no-allocation write-back is
    refused (its destinations are host slots); a load into the small device
    pool still runs."""
    S_host = (1 << 24) + 16
    g = Geometry(1, 1, 16, 4096, S_host, 16, oracle.LAYER_FIRST)
    bufs = device_buffers(g, seed=13, fill=9)
    pool = kvt.KvPool(kv_geom(g), bufs)
    s = torch.cuda.Stream()
    idx = np.arange(4, dtype=np.int64)
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.BACKUP, idx, idx, 0, 1, s) == kvt.EINVAL
    assert "2^24" in kvt.kv_last_error()
    assert kvt.kv_transfer_noalloc(pool.handle, kvt.LOAD, idx, idx + S_host - 4, 0, 1, s) == kvt.OK
    s.synchronize()
    pool.close()
