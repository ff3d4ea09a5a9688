"""The library's Ghost List (kv_page_hashes, kv_ghost_*) against the oracle,
element by element: page-boundary hashes of random token sequences, and the
list's contents in order, size, membership and proven-reuse prefixes after
every operation of random operation streams. Host-only: no GPU needed."""
import ctypes
import threading

import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
from oracle import ghost


@pytest.mark.parametrize("ps", [1, 3, 16, 64])
def test_page_hashes_match_oracle(ps):
    rng = np.random.default_rng(ps)
    for n in (0, 1, ps - 1, ps, 5 * ps + 1, 7 * ps):
        if n < 0:
            continue
        t = rng.integers(-2**31, 2**31, size=n, dtype=np.int64).astype(np.int32)
        got = [int(x) for x in kvt.kv_page_hashes(t, ps)]
        assert got == ghost.page_hashes(t.tolist(), ps), (ps, n)


def test_page_hashes_rejects_bad_arguments():
    lib = kvt.library()
    t = np.zeros(8, np.int32)
    out = np.zeros(8, np.uint64)
    tp = t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    op = out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    assert lib.kv_page_hashes(tp, 8, 0, op) == kvt.EINVAL
    assert lib.kv_page_hashes(tp, -1, 4, op) == kvt.EINVAL
    assert lib.kv_page_hashes(None, 8, 4, op) == kvt.EINVAL
    assert lib.kv_page_hashes(None, 3, 4, None) == 0       # no full page: nothing read


def _compare(lib_g, ora_g):
    assert lib_g.order() == ora_g.order()
    assert lib_g.size() == ora_g.size()


@pytest.mark.parametrize("cap,keys", [(1, 4), (2, 6), (3, 16), (8, 20), (64, 200), (64, 1 << 62)])
def test_operation_streams_match_oracle(cap, keys):
    rng = np.random.default_rng(cap * 7 + (keys % 1000))
    lg, og = kvt.GhostList(cap), ghost.GhostList(cap)
    for step in range(400):
        hs = rng.integers(0, keys, size=int(rng.integers(0, 2 * cap + 2)), dtype=np.int64)
        hs = [int(x) for x in hs]
        lg.insert(hs)
        og.insert(hs)
        _compare(lg, og)
        q = [int(x) for x in rng.integers(0, keys, size=int(rng.integers(0, 10)), dtype=np.int64)]
        assert lg.reuse_prefix(q) == og.reuse_prefix(q)
        for x in q[:3]:
            assert lg.contains(x) == og.contains(x)
    lg.close()


def test_full_64_bit_keys_and_scale():
    """65,536 entries, 300,000 inserts of random 64-bit page hashes with repeats."""
    rng = np.random.default_rng(5)
    cap = 1 << 16
    pool = rng.integers(0, 2**63, size=200_000, dtype=np.int64).astype(np.uint64) * np.uint64(2) \
        + rng.integers(0, 2, size=200_000, dtype=np.int64).astype(np.uint64)
    stream = pool[rng.integers(0, pool.size, size=300_000)]
    lg, og = kvt.GhostList(cap), ghost.GhostList(cap)
    for chunk in np.array_split(stream, 30):
        lg.insert(chunk)
        og.insert(chunk.tolist())
    _compare(lg, og)
    for _ in range(50):
        q = pool[rng.integers(0, pool.size, size=64)]
        assert lg.reuse_prefix(q) == og.reuse_prefix(q.tolist())
    lg.close()


def test_page_hashes_through_the_list():
    """The rebuild scenario with hashes from the library: evict one request's
    pages, rebuild requests that share 0, 6 and 8 of its 10 pages."""
    ps = 64
    rng = np.random.default_rng(6)
    a = rng.integers(0, 150000, size=10 * ps, dtype=np.int64).astype(np.int32)
    g = kvt.GhostList(1024)
    g.insert(kvt.kv_page_hashes(a, ps))
    for share in (0, 6, 8, 10):
        b = np.concatenate([a[:share * ps], rng.integers(150000, 160000, size=(10 - share) * ps,
                                                         dtype=np.int64).astype(np.int32)])
        assert g.reuse_prefix(kvt.kv_page_hashes(b, ps)) == share
    g.close()


def test_create_and_call_errors():
    assert kvt.kv_ghost_create(0)[0] == kvt.EINVAL
    assert kvt.kv_ghost_create(-5)[0] == kvt.EINVAL
    assert kvt.kv_ghost_create((1 << 30) + 1)[0] == kvt.EINVAL
    lib = kvt.library()
    assert lib.kv_ghost_insert(None, None, 0) == kvt.EINVAL
    assert lib.kv_ghost_reuse_prefix(None, None, 0) == kvt.EINVAL
    assert lib.kv_ghost_size(None) == kvt.EINVAL
    g = kvt.GhostList(4)
    assert lib.kv_ghost_insert(g.handle, None, 3) == kvt.EINVAL
    assert lib.kv_ghost_insert(g.handle, None, -1) == kvt.EINVAL
    assert lib.kv_ghost_reuse_prefix(g.handle, None, 2) == kvt.EINVAL
    assert lib.kv_ghost_insert(g.handle, None, 0) == kvt.OK
    assert lib.kv_ghost_reuse_prefix(g.handle, None, 0) == 0
    assert kvt.kv_ghost_destroy(None) == kvt.OK
    g.close()


def test_concurrent_inserts():
    """Four threads insert disjoint key sets into a list large enough for all:
    every key is present afterwards, each thread's keys in its own order."""
    g = kvt.GhostList(4 * 5000)
    sets = [np.arange(k * 10**6, k * 10**6 + 5000, dtype=np.uint64) for k in range(4)]

    def run(keys):
        for c in np.array_split(keys, 50):
            g.insert(c)

    th = [threading.Thread(target=run, args=(s,)) for s in sets]
    for x in th:
        x.start()
    for x in th:
        x.join()
    order = g.order()
    assert g.size() == 20000 and len(order) == 20000
    for s in sets:
        mine = [h for h in order if s[0] <= h <= s[-1]]
        assert mine == [int(x) for x in s]
    g.close()
