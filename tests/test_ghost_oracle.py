"""Pins of the Ghost List oracle (oracle/ghost.py) against what the pages and
the hash's published definition fix, independent of the oracle's own code:
published FNV-1a test vectors, the hash's streaming property, prefix and
position behaviour of page-boundary hashes, least-recently-inserted eviction
against a plain list model, and the backward scan against a brute-force
maximum. Source: "Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section
2.6; "Baidu's KVCache Overhaul", "write_through_selective with Ghost List"."""
import json
import os

import numpy as np
import pytest

from oracle import ghost

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fnv1a64_published_vectors():
    spec = json.load(open(os.path.join(HERE, "golden", "fnv1a64.json")))
    for v in spec["vectors"]:
        assert ghost.fnv1a64(v["input"].encode()) == int(v["fnv1a64"], 16), v


def test_fnv1a64_streams():
    rng = np.random.default_rng(0)
    for _ in range(20):
        a = bytes(rng.integers(0, 256, size=int(rng.integers(0, 40)), dtype=np.uint8))
        b = bytes(rng.integers(0, 256, size=int(rng.integers(0, 40)), dtype=np.uint8))
        assert ghost.fnv1a64(b, ghost.fnv1a64(a)) == ghost.fnv1a64(a + b)


def test_token_encoding():
    assert ghost.page_hashes([1], 1) == [ghost.fnv1a64(b"\x01\x00\x00\x00")]
    assert ghost.page_hashes([-1, 258], 2) == [ghost.fnv1a64(b"\xff\xff\xff\xff\x02\x01\x00\x00")]


def test_partial_page_has_no_hash():
    t = list(range(10))
    assert len(ghost.page_hashes(t, 4)) == 2
    assert ghost.page_hashes(t[:3], 4) == []
    assert ghost.page_hashes([], 4) == []
    assert ghost.page_hashes(t, 4) == ghost.page_hashes(t[:8], 4)


def test_shared_prefix_shares_leading_hashes():
    rng = np.random.default_rng(1)
    ps = 4
    a = rng.integers(0, 50000, size=40).tolist()
    for j in range(10):                      # first differing page
        b = list(a)
        b[j * ps + int(rng.integers(0, ps))] += 1
        ha, hb = ghost.page_hashes(a, ps), ghost.page_hashes(b, ps)
        assert ha[:j] == hb[:j]
        assert all(x != y for x, y in zip(ha[j:], hb[j:]))


def test_hash_names_position():
    page = [7, 8, 9, 10]
    h1 = ghost.page_hashes(page, 4)
    h2 = ghost.page_hashes([1, 2, 3, 4] + page, 4)
    assert h1[0] != h2[1]                     # same content, another position


class NaiveLRU:
    """Plain list, least recent first."""

    def __init__(self, cap):
        self.cap, self.items = cap, []

    def insert(self, hs):
        for h in hs:
            if h in self.items:
                self.items.remove(h)
            elif len(self.items) == self.cap:
                self.items.pop(0)
            self.items.append(h)


@pytest.mark.parametrize("cap", [1, 2, 3, 5, 8])
def test_eviction_order_matches_list_model(cap):
    rng = np.random.default_rng(cap)
    g, m = ghost.GhostList(cap), NaiveLRU(cap)
    for _ in range(300):
        hs = rng.integers(0, 12, size=int(rng.integers(0, 5))).tolist()
        g.insert(hs)
        m.insert(hs)
        assert g.order() == m.items
        q = int(rng.integers(0, 12))
        assert g.contains(q) == (q in m.items)
        assert g.size() == len(m.items) <= cap


def test_lookup_keeps_order_and_reinsert_refreshes():
    g = ghost.GhostList(2)
    g.insert([1, 2])
    assert g.contains(1) and g.reuse_prefix([1]) == 1
    g.insert([3])                             # 1 is still the least recent
    assert g.order() == [2, 3]
    g.insert([2, 4])                          # 2 refreshed, 3 dropped
    assert g.order() == [2, 4]


def test_reuse_prefix_is_the_last_hit():
    rng = np.random.default_rng(2)
    for _ in range(200):
        g = ghost.GhostList(int(rng.integers(1, 20)))
        g.insert(rng.integers(0, 30, size=int(rng.integers(0, 30))).tolist())
        hs = rng.integers(0, 30, size=int(rng.integers(0, 12))).tolist()
        want = max([k + 1 for k, h in enumerate(hs) if h in set(g.order())], default=0)
        assert g.reuse_prefix(hs) == want


def test_rebuild_scenario():
    """Request A's ten pages leave L1; B shares A's first six pages, C nothing,
    D eight pages; with room for only four ghosts, only A's last four remain."""
    ps = 16
    rng = np.random.default_rng(3)
    a = rng.integers(0, 32000, size=10 * ps).tolist()
    b = a[:6 * ps] + rng.integers(0, 32000, size=4 * ps).tolist()
    c = rng.integers(0, 32000, size=5 * ps).tolist()
    d = a[:8 * ps] + rng.integers(0, 32000, size=2 * ps).tolist()
    ha = ghost.page_hashes(a, ps)
    big = ghost.GhostList(100)
    big.insert(ha)
    assert big.reuse_prefix(ghost.page_hashes(b, ps)) == 6
    assert big.reuse_prefix(ghost.page_hashes(c, ps)) == 0
    assert big.reuse_prefix(ghost.page_hashes(d, ps)) == 8
    small = ghost.GhostList(4)
    small.insert(ha)
    assert small.order() == ha[6:]
    assert small.reuse_prefix(ghost.page_hashes(b, ps)) == 0
    assert small.reuse_prefix(ghost.page_hashes(d, ps)) == 8
