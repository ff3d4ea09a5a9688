"""Concurrent write-back and load on one pool, and the landed events of loads
on several streams, through the C ABI.

* Every (write-back path x load path) pairing, and AUTO on a pool flagged
  KV_F_DUPLEX, runs a write-back and a load from two threads on two streams at
  once against one pool; the whole host pool and every device buffer must
  equal the oracle's, which runs the two transfers one after the other (they
  touch disjoint rows). The dedicated backup and load threads on private
  streams are the pages' bidirectional submission ("Tuning SGLang HiCache L2
  on Kunlunxin P800/P900", section 2.2; "Baidu's KVCache Overhaul",
  "Bidirectional Async Transfer").
* A load that covers every layer in one group, held back on its stream, and a
  later load on another stream that covers only the first layers: a consumer
  gated with kv_load_layer on a layer only the first load covers must see that
  load's bytes.
"""
import threading

import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
import oracle
from oracle import Geometry

from gpu_util import SENTINEL, device_buffers, kv_geom, mirrors, torch_mod

pytestmark = pytest.mark.gpu

DIRECT = (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS, kvt.PATH_DMA, kvt.PATH_STAGED)
NAMES = {kvt.PATH_KERNEL: "kernel", kvt.PATH_KERNEL_LDS: "lds", kvt.PATH_DMA: "dma",
         kvt.PATH_STAGED: "staged", kvt.PATH_AUTO: "auto"}
LAYOUTS = (oracle.LAYER_FIRST, oracle.PAGE_FIRST, oracle.PAGE_FIRST_DIRECT)


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def _split(g, seed):
    """Disjoint request sets of one pool: `load` reads host pages into device
    slots, `back` writes other device slots to other host pages. Pages are
    whole and in random order on both sides, with a ragged last page on the
    write-back."""
    rng = np.random.default_rng(seed)
    ps = g.ps
    dev_pages = rng.permutation(g.S_dev // ps)
    host_pages = rng.permutation(g.S_host // ps)
    n_load, n_back = 5, 4
    tok = lambda pages: (pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
    ld = tok(dev_pages[:n_load])
    lh = tok(host_pages[:n_load])
    bd = tok(dev_pages[n_load:n_load + n_back])[:n_back * ps - ps // 2]
    bh = tok(host_pages[n_load:n_load + n_back])[:n_back * ps - ps // 2]
    return ld.astype(np.int64), lh.astype(np.int64), bd.astype(np.int64), bh.astype(np.int64)


def _run_concurrently(fns):
    go = threading.Barrier(len(fns))
    errors = []

    def run(fn):
        try:
            go.wait()
            fn()
        except Exception as e:  # surfaced below
            errors.append(e)

    th = [threading.Thread(target=run, args=(fn,)) for fn in fns]
    for x in th:
        x.start()
    for x in th:
        x.join()
    assert not errors, errors


PAIRS = [(b, l) for b in DIRECT for l in DIRECT] + [(kvt.PATH_AUTO, kvt.PATH_AUTO)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("back_path,load_path", PAIRS,
                         ids=["%s-%s" % (NAMES[b], NAMES[l]) for b, l in PAIRS])
def test_duplex_pairing_whole_pool(torch, layout, back_path, load_path):
    g = Geometry(4, 2, 272, 1024, 768, 16, layout)
    print("duplex pairing back=%s load=%s layout=%d" % (NAMES[back_path], NAMES[load_path],
                                                        layout), flush=True)
    bufs = device_buffers(g, seed=40 + layout)
    flags = kvt.F_CHECK_UNIQUE | (kvt.F_DUPLEX if back_path == kvt.PATH_AUTO else 0)
    pool = kvt.KvPool(kv_geom(g), bufs, flags=flags)
    pool.set_path(back_path, kvt.BACKUP)
    pool.set_path(load_path, kvt.LOAD)
    host = pool.host_array()
    host[:] = np.random.default_rng(50 + layout).integers(0, 256, host.size, dtype=np.uint8)
    ld, lh, bd, bh = _split(g, 60 + layout)
    want_host = host.copy()
    want_dev = mirrors(bufs)
    assert oracle.backup(g, want_dev, want_host, bd, bh) == 0
    assert oracle.load(g, want_dev, want_host, ld, lh) == 0
    s_back, s_load = kvt.Stream(), kvt.Stream()
    _run_concurrently([lambda: pool.backup(bd, bh, 0, g.L, s_back),
                       lambda: pool.load(ld, lh, 0, g.L, s_load)])
    s_back.synchronize()
    s_load.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(pool.host_array(), want_host)
    for k, b in enumerate(bufs):
        assert np.array_equal(b.cpu().numpy(), want_dev[k]), k
    if back_path != kvt.PATH_AUTO:
        assert pool.last_path(kvt.BACKUP) == back_path
        assert pool.last_path(kvt.LOAD) == load_path
    s_back.close()
    s_load.close()
    pool.close()


def test_direction_path_is_per_direction(torch):
    g = Geometry(2, 1, 64, 64, 64, 8, 0)
    bufs = device_buffers(g, seed=7)
    pool = kvt.KvPool(kv_geom(g), bufs)
    pool.set_path(kvt.PATH_DMA, kvt.BACKUP)
    pool.set_path(kvt.PATH_KERNEL, kvt.LOAD)
    s = torch.cuda.Stream()
    idx = np.arange(16)
    pool.backup(idx, idx, 0, 2, s)
    pool.load(idx + 16, idx, 0, 2, s)
    s.synchronize()
    assert pool.last_path(kvt.BACKUP) == kvt.PATH_DMA
    assert pool.last_path(kvt.LOAD) == kvt.PATH_KERNEL
    assert kvt.kv_set_direction_path(pool.handle, 2, kvt.PATH_DMA) == kvt.EINVAL
    assert kvt.kv_set_direction_path(pool.handle, 0, 9) == kvt.EINVAL
    assert kvt.kv_set_direction_path(None, 0, kvt.PATH_DMA) == kvt.EINVAL
    pool.close()


@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED))
def test_landed_event_survives_a_partial_load_on_another_stream(torch, path):
    """Load A covers all 8 layers in one group on stream s1, queued behind
    ~20 passes over a 1 GiB tensor; load B then covers layers [0, 2) at other
    slots on stream s2 and lands at once. A consumer on s3 gated by
    kv_load_layer(5) must read A's layer 5, although B's group starts at the
    layer A's group started at."""
    L, C, R, n = 8, 2, 256, 512
    g = Geometry(L, C, R, 4 * n, 2 * n, 16, oracle.LAYER_FIRST)
    bufs = device_buffers(g, seed=11, fill=0)
    pool = kvt.KvPool(kv_geom(g), bufs)
    pool.set_path(path)
    host = pool.host_array()
    host[:] = np.random.default_rng(12).integers(0, 256, host.size, dtype=np.uint8)
    c = pool.calibration()
    c.load_split_min_bytes = 64.0 * 1024 * 1024     # one group for each load
    pool.set_calibration(c)
    a_dev, b_dev = np.arange(n), np.arange(2 * n, 3 * n)
    a_host, b_host = np.arange(n), np.arange(n, 2 * n)
    want = [int(oracle_rows(g, host, l, cc, a_host).astype(np.int64).sum())
            for l in range(L) for cc in range(C)]
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    big = torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    print("partial-range landed events path=%d" % path, flush=True)
    with torch.cuda.stream(s1):
        for _ in range(20):
            big.add_(1.0)                       # hold s1 for a few milliseconds
    pool.load(a_dev, a_host, 0, L, s1)
    pool.load(b_dev, b_host, 0, 2, s2)
    with torch.cuda.stream(s3):
        sums = torch.zeros(C, dtype=torch.int64, device="cuda:0")
        pool.load_layer(5, s3)
        for cc in range(C):
            sums[cc] = bufs[5 * C + cc].view(-1, R)[:n].to(torch.int64).sum()
    s3.synchronize()
    s1.synchronize()
    s2.synchronize()
    got = [int(x) for x in sums.cpu()]
    assert got == want[5 * C:6 * C], (got, want[5 * C:6 * C])
    pool.close()


def oracle_rows(g, host, l, c, h):
    """Host rows (l, c, h[i]) through the oracle's address map, as (n, R)."""
    rows = [oracle.host_row(g, l, c, int(x)) for x in h]
    return np.stack([host[r * g.R:(r + 1) * g.R] for r in rows])
