"""The write-through-selective filter deciding what a write-back moves, end to
end on the GPU ("Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.6,
"Write-policy semantic fix + Ghost List"; "Baidu's KVCache Overhaul",
"write_through_selective with Ghost List").

Requests whose pages left the device pool have their page-boundary hashes in a
bounded Ghost List. Rebuilt requests share 0 to all of an evicted request's
pages; each one's hashes are scanned for the longest proven-reuse prefix, and
exactly that prefix's pages are written back with kv_backup. The library side
(kv_page_hashes, kv_ghost_*, kv_backup on the GPU) and the oracle side
(oracle.ghost, then the C oracle's backup on host mirrors) each take their own
decisions; the decisions and the whole host pool, untouched sentinel bytes
included, must be equal.
"""
import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
import oracle
from oracle import Geometry, ghost

from gpu_util import PATHS, SENTINEL, device_buffers, kv_geom, mirrors, torch_mod

pytestmark = pytest.mark.gpu

PS = 16
PAGES = 12


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def scenario(seed):
    """Evicted requests (token lists) and rebuilt requests sharing a prefix of
    the first evicted one, with the device pages each rebuilt request's KV
    occupies and the host pages its write-back may use."""
    rng = np.random.default_rng(seed)
    evicted = [rng.integers(0, 150000, size=PAGES * PS).astype(np.int32) for _ in range(3)]
    rebuilt = []
    for k, share in enumerate((0, 3, 7, PAGES, 5)):
        tail = rng.integers(150000, 160000, size=(PAGES - share) * PS).astype(np.int32)
        src = evicted[0] if k != 4 else evicted[2]
        rebuilt.append(np.concatenate([src[:share * PS], tail]))
    dev_pages = rng.permutation(128)[:len(rebuilt) * PAGES].reshape(len(rebuilt), PAGES)
    host_pages = rng.permutation(64)[:len(rebuilt) * PAGES].reshape(len(rebuilt), PAGES)
    return evicted, rebuilt, dev_pages, host_pages


def tokens_of(pages):
    pages = np.asarray(pages, dtype=np.int64)
    return (pages[:, None] * PS + np.arange(PS)[None, :]).reshape(-1)


@pytest.mark.parametrize("layout", (oracle.LAYER_FIRST, oracle.PAGE_FIRST,
                                    oracle.PAGE_FIRST_DIRECT))
@pytest.mark.parametrize("path", PATHS)
def test_ghost_list_decides_the_write_back(torch, layout, path):
    g = Geometry(4, 2, 256, 128 * PS, 64 * PS, PS, layout)
    evicted, rebuilt, dev_pages, host_pages = scenario(70 + layout)
    print("ghost write-back layout=%d path=%d" % (layout, path), flush=True)
    # a list that holds 30 hashes: of 36 evicted pages the first 6 inserted are
    # dropped again, so a prefix sharing up to 6 pages of the first request is
    # no longer proven
    lib_list, ora_list = kvt.GhostList(30), ghost.GhostList(30)
    for toks in evicted:
        lib_list.insert(kvt.kv_page_hashes(toks, PS))
        ora_list.insert(ghost.page_hashes(toks.tolist(), PS))
    assert lib_list.order() == ora_list.order()

    bufs = device_buffers(g, seed=80 + layout)
    pool = kvt.KvPool(kv_geom(g), bufs)
    pool.set_path(path)
    pool.host_array()[:] = SENTINEL
    want = np.full(g.host_bytes(), SENTINEL, np.uint8)
    dev_m = mirrors(bufs)
    s = torch.cuda.Stream()
    decided = []
    for toks, dpages, hpages in zip(rebuilt, dev_pages, host_pages):
        k_lib = lib_list.reuse_prefix(kvt.kv_page_hashes(toks, PS))
        k_ora = ora_list.reuse_prefix(ghost.page_hashes(toks.tolist(), PS))
        assert k_lib == k_ora
        decided.append(k_ora)
        if k_lib:
            pool.backup(tokens_of(dpages[:k_lib]), tokens_of(hpages[:k_lib]), 0, g.L, s)
        if k_ora:
            assert oracle.backup(g, dev_m, want, tokens_of(dpages[:k_ora]),
                                 tokens_of(hpages[:k_ora])) == 0
    s.synchronize()
    torch.cuda.synchronize()
    # shares 0, 3, 7, 12 of the first evicted request and 5 of the third: the
    # first request's pages 1-6 were dropped, so 3 pages prove nothing
    assert decided == [0, 0, 7, PAGES, 5]
    got = pool.host_array()
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        raise AssertionError("host pool differs at %d bytes, first at %d" % (bad.size, bad[0]))
    lib_list.close()
    pool.close()
