"""Helpers shared by the GPU tests: device pools from torch, host mirrors for the
oracle, and byte comparisons. Every transfer goes through the C ABI."""
import numpy as np

import hierarchical_kv_cache_backup_amd as kvt
import oracle
from oracle import Geometry

SENTINEL = 0xA5
PATHS = (kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS, kvt.PATH_DMA, kvt.PATH_STAGED, kvt.PATH_AUTO)


def torch_mod():
    import torch
    return torch


def device_buffers(g, seed, fill=None):
    """L*C uint8 device tensors of S_dev*R bytes: seeded random bytes (made on the
    CPU so the oracle sees the same values) or a constant fill."""
    torch = torch_mod()
    bufs = []
    rng = np.random.default_rng(seed)
    for _ in range(g.L * g.C):
        if fill is None:
            a = rng.integers(0, 256, size=g.S_dev * g.R, dtype=np.uint8)
            bufs.append(torch.from_numpy(a).to("cuda:0"))
        else:
            bufs.append(torch.full((g.S_dev * g.R,), fill, dtype=torch.uint8, device="cuda:0"))
    return bufs


def mirrors(bufs):
    return [b.cpu().numpy().copy() for b in bufs]


def kv_geom(g):
    return kvt.geometry(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout)


def make_pool(g, bufs, path=kvt.PATH_KERNEL, flags=kvt.F_CHECK_UNIQUE, host_fill=SENTINEL):
    pool = kvt.KvPool(kv_geom(g), bufs, device=0, flags=flags)
    pool.set_path(path)
    if host_fill is not None:
        pool.host_array()[:] = host_fill
    return pool


def run_backup_and_compare(g, pool, bufs, d, h, l0, l1, stream):
    """kv_backup on the GPU; the oracle on mirrors; the whole host pool must match."""
    torch = torch_mod()
    want = pool.host_array().copy()
    dev_m = mirrors(bufs)
    assert oracle.backup(g, dev_m, want, d, h, l0, l1) == 0
    pool.backup(d, h, l0, l1, stream)
    stream.synchronize()
    torch.cuda.synchronize()
    got = pool.host_array()
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError("host pool differs at %d bytes, first at %d" % (bad.size, bad[0]))


def run_load_and_compare(g, pool, bufs, d, h, l0, l1, stream):
    """kv_load on the GPU; the oracle on mirrors; every device buffer must match."""
    torch = torch_mod()
    host = pool.host_array().copy()
    dev_m = mirrors(bufs)
    assert oracle.load(g, dev_m, host, d, h, l0, l1) == 0
    pool.load(d, h, l0, l1, stream)
    stream.synchronize()
    torch.cuda.synchronize()
    for k, b in enumerate(bufs):
        got = b.cpu().numpy()
        if not np.array_equal(got, dev_m[k]):
            bad = np.flatnonzero(got != dev_m[k])
            raise AssertionError("device buffer %d differs at %d bytes, first at %d"
                                 % (k, bad.size, bad[0]))
