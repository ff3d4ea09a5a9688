"""Pins of the CPU oracle against what the pages and plain arithmetic fix.

Nothing here compares the oracle with itself: every check reaches the expected
value another way (the pages' printed example, hand-enumerated storage orders,
a NumPy derivation by reshape/transpose, closed forms, special cases that reduce
to a slice copy, brute force over all permutations of tiny requests).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import np_ref
from oracle import Geometry, LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT, LAYOUTS

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")
LAYOUT_BY_NAME = {"layer_first": LAYER_FIRST, "page_first": PAGE_FIRST,
                  "page_first_direct": PAGE_FIRST_DIRECT}
SENTINEL = 0xA5


def parse_layout_golden():
    sections = {}
    cur = None
    with open(os.path.join(GOLDEN, "layout_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                kv = dict(tok.split("=") for tok in line.strip("[]").split()[1:])
                cur = (int(kv["L"]), int(kv["C"]), int(kv["S_host"]), int(kv["ps"]))
                sections[cur] = []
                continue
            name, row, l, c, h = line.split()
            sections[cur].append((LAYOUT_BY_NAME[name], int(row), int(l), int(c), int(h)))
    return sections


# ---- helpers ----------------------------------------------------------------

def random_pool(rng, g):
    """L*C device mirrors with random bytes, stacked view, and a sentinel host pool."""
    dev = rng.integers(0, 256, size=(g.L, g.C, g.S_dev, g.R), dtype=np.uint8)
    host = np.full(g.host_bytes(), SENTINEL, dtype=np.uint8)
    return dev, host


def bufs_of(dev):
    return [np.array(dev[l, c], copy=True).reshape(-1) for l in range(dev.shape[0])
            for c in range(dev.shape[1])]


def stack_bufs(bufs, g):
    return np.stack([b.reshape(g.S_dev, g.R) for b in bufs]).reshape(g.L, g.C, g.S_dev, g.R)


def oracle_backup(g, dev, host, d, h, l0=0, l1=None, o=None):
    o = o or oracle.default()
    bufs = bufs_of(dev)
    rc = o.backup(g, bufs, host, d, h, l0, l1)
    return rc


def oracle_load(g, dev, host, d, h, l0=0, l1=None, o=None):
    """Returns (rc, new stacked device array)."""
    o = o or oracle.default()
    bufs = bufs_of(dev)
    rc = o.load(g, bufs, host, d, h, l0, l1)
    return rc, stack_bufs(bufs, g)


def random_request(rng, g, n, direction_unique="both"):
    d = rng.choice(g.S_dev, size=n, replace=False).astype(np.int64)
    h = rng.choice(g.S_host, size=n, replace=False).astype(np.int64)
    return d, h


def random_geometry(rng, layout=None):
    L = int(rng.integers(1, 5))
    C = int(rng.integers(1, 3))
    R = 16 * int(rng.integers(1, 4))
    ps = int(rng.choice([1, 2, 3, 4, 8]))
    S_host = ps * int(rng.integers(1, 9))
    S_dev = int(rng.integers(max(1, S_host // 2), S_host + 12))
    layout = int(rng.integers(0, 3)) if layout is None else layout
    return Geometry(L, C, R, S_dev, S_host, ps, layout)


# ---- 1. the pages' storage orders, enumerated by hand -------------------------

def test_golden_storage_orders_match_oracle_and_numpy():
    sections = parse_layout_golden()
    assert len(sections) == 2
    for (L, C, S_host, ps), rows in sections.items():
        for layout in LAYOUTS:
            lines = [r for r in rows if r[0] == layout]
            assert len(lines) == L * C * S_host
            assert sorted(r[1] for r in lines) == list(range(L * C * S_host))
            g = Geometry(L, C, 16, S_host, S_host, ps, layout)
            table = np_ref.row_id_table(layout, L, C, S_host, ps)
            for _, row, l, c, h in lines:
                assert oracle.host_row(g, l, c, h) == row, (layout, l, c, h)
                assert table[l, c, h] == row


def test_pages_segment_count_example():
    """512 pages x 78 layers = 39,936 segments for page_first_direct, 78 for layer_first."""
    with open(os.path.join(GOLDEN, "segment_counts.json")) as f:
        gold = json.load(f)
    n, ps, L, C = gold["tokens"], gold["page_size"], gold["layers"], gold["components"]
    d = np.arange(n, dtype=np.int64) + 4096        # contiguous device slots
    h = np.arange(n, dtype=np.int64)                # host slots from a page boundary
    for layout, key in ((PAGE_FIRST_DIRECT, "page_first_direct_segments"),
                        (LAYER_FIRST, "layer_first_segments")):
        g = Geometry(L, C, gold["row_bytes"], 65536, n, ps, layout)
        assert oracle.count_segments(g, d, h) == gold[key]
        assert np_ref.count_segments(layout, L, C, n, ps, d, h) == gold[key]


# ---- 2. closed forms ----------------------------------------------------------

@pytest.mark.parametrize("seed", range(12))
def test_segment_closed_forms_contiguous(seed):
    rng = np.random.default_rng(seed)
    L, C, ps = int(rng.integers(1, 6)), int(rng.integers(1, 3)), int(rng.choice([1, 2, 4, 16]))
    pages = int(rng.integers(1, 9))
    n = pages * ps
    S_host = n + ps * int(rng.integers(0, 3))
    h0 = ps * int(rng.integers(0, (S_host - n) // ps + 1))
    d0 = int(rng.integers(0, 50))
    d = np.arange(d0, d0 + n, dtype=np.int64)
    h = np.arange(h0, h0 + n, dtype=np.int64)
    l0 = int(rng.integers(0, L))
    l1 = int(rng.integers(l0, L + 1))
    nl = l1 - l0
    expect = {LAYER_FIRST: nl * C,
              PAGE_FIRST_DIRECT: nl * C * pages if L * C > 1 else nl * C,
              PAGE_FIRST: nl * C * n if L * C > 1 else nl * C}
    for layout in LAYOUTS:
        g = Geometry(L, C, 16, d0 + n, S_host, ps, layout)
        assert oracle.count_segments(g, d, h, l0, l1) == expect[layout], layout


@pytest.mark.parametrize("seed", range(8))
def test_layer_first_segments_count_breaks(seed):
    """layer_first: every (l, c) has 1 + (#positions where device or host slot jumps)."""
    rng = np.random.default_rng(100 + seed)
    L, C = int(rng.integers(1, 5)), int(rng.integers(1, 3))
    n = int(rng.integers(1, 40))
    d = rng.choice(200, size=n, replace=False).astype(np.int64)
    h = rng.choice(200, size=n, replace=False).astype(np.int64)
    if seed % 2:
        d = np.sort(d)
        h = np.sort(h)
    breaks = sum(1 for i in range(1, n) if not (d[i] == d[i - 1] + 1 and h[i] == h[i - 1] + 1))
    g = Geometry(L, C, 32, 200, 200, 4, LAYER_FIRST)
    assert oracle.count_segments(g, d, h) == L * C * (1 + breaks)


# ---- 3. NumPy derivation == oracle (random requests, all layouts) ---------------

@pytest.mark.parametrize("seed", range(40))
def test_oracle_matches_numpy_derivation(seed):
    rng = np.random.default_rng(1000 + seed)
    g = random_geometry(rng)
    n = int(rng.integers(0, min(g.S_dev, g.S_host) + 1))
    d, h = random_request(rng, g, n)
    l0 = int(rng.integers(0, g.L + 1))
    l1 = int(rng.integers(l0, g.L + 1))
    dev, host = random_pool(rng, g)
    # backup
    host_np = host.copy()
    np_ref.backup(dev, host_np, g.layout, g.L, g.C, g.S_host, g.ps, g.R, d, h, l0, l1)
    assert oracle_backup(g, dev, host, d, h, l0, l1) == oracle.OK
    assert np.array_equal(host, host_np)
    # load from a random host image into the device pool
    src = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
    dev_np = dev.copy()
    np_ref.load(dev_np, src, g.layout, g.L, g.C, g.S_host, g.ps, g.R, d, h, l0, l1)
    rc, dev_or = oracle_load(g, dev, src, d, h, l0, l1)
    assert rc == oracle.OK
    assert np.array_equal(dev_or, dev_np)
    # segment counts agree with the table-based counter
    assert oracle.count_segments(g, d, h, l0, l1) == np_ref.count_segments(
        g.layout, g.L, g.C, g.S_host, g.ps, d, h, l0, l1)


# ---- 4. round trip, untouched bytes, layer range ---------------------------------

@pytest.mark.parametrize("layout", LAYOUTS)
def test_round_trip_identity_and_sentinels(layout):
    rng = np.random.default_rng(7)
    g = Geometry(3, 2, 48, 40, 32, 4, layout)
    dev, host = random_pool(rng, g)
    n = 20
    d1 = rng.choice(g.S_dev, n, replace=False)
    h = rng.choice(g.S_host, n, replace=False)
    d2 = rng.choice(g.S_dev, n, replace=False)
    assert oracle_backup(g, dev, host, d1, h) == oracle.OK
    fresh = np.full_like(dev, SENTINEL)
    rc, out = oracle_load(g, fresh, host, d2, h)
    assert rc == oracle.OK
    for l in range(g.L):
        for c in range(g.C):
            assert np.array_equal(out[l, c, d2], dev[l, c, d1])
            untouched = np.setdiff1d(np.arange(g.S_dev), d2)
            assert (out[l, c, untouched] == SENTINEL).all()
    # host rows not written keep the sentinel
    touched = np.zeros(g.L * g.C * g.S_host, bool)
    for l in range(g.L):
        for c in range(g.C):
            for hh in h:
                touched[oracle.host_row(g, l, c, hh)] = True
    rows = host.reshape(-1, g.R)
    assert (rows[~touched] == SENTINEL).all()
    assert not (rows[touched] == SENTINEL).all(axis=1).any()


def test_round_trip_is_layout_independent():
    rng = np.random.default_rng(8)
    base = Geometry(4, 2, 32, 50, 48, 8, LAYER_FIRST)
    dev, _ = random_pool(rng, base)
    n = 30
    d1 = rng.choice(base.S_dev, n, replace=False)
    h = rng.choice(base.S_host, n, replace=False)
    d2 = rng.choice(base.S_dev, n, replace=False)
    outs = []
    for layout in LAYOUTS:
        g = base.replace(layout=layout)
        host = np.full(g.host_bytes(), SENTINEL, np.uint8)
        oracle_backup(g, dev, host, d1, h)
        _, out = oracle_load(g, np.full_like(dev, SENTINEL), host, d2, h)
        outs.append(out)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_layers_outside_range_untouched(layout):
    rng = np.random.default_rng(9)
    g = Geometry(5, 2, 32, 20, 16, 4, layout)
    dev, host = random_pool(rng, g)
    d = rng.choice(g.S_dev, 10, replace=False)
    h = rng.choice(g.S_host, 10, replace=False)
    oracle_backup(g, dev, host, d, h, 1, 3)
    rows = host.reshape(-1, g.R)
    for l in range(g.L):
        for c in range(g.C):
            for hh in h:
                r = oracle.host_row(g, l, c, hh)
                if 1 <= l < 3:
                    assert np.array_equal(rows[r], dev[l, c, d[list(h).index(hh)]])
                else:
                    assert (rows[r] == SENTINEL).all()
    src = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
    _, out = oracle_load(g, dev, src, d, h, 2, 5)
    assert np.array_equal(out[:2], dev[:2])


# ---- 5. degenerate cases that reduce to simpler definitions ----------------------

def test_single_buffer_maps_are_identity():
    """L = C = 1: every layout stores slot h at row h."""
    for layout in LAYOUTS:
        g = Geometry(1, 1, 16, 64, 64, 8, layout)
        assert [oracle.host_row(g, 0, 0, h) for h in range(64)] == list(range(64))


def test_page_size_one_direct_equals_page_first():
    for L, C in ((3, 2), (2, 1), (5, 2)):
        a = Geometry(L, C, 16, 8, 12, 1, PAGE_FIRST_DIRECT)
        b = a.replace(layout=PAGE_FIRST)
        for l in range(L):
            for c in range(C):
                for h in range(12):
                    assert oracle.host_row(a, l, c, h) == oracle.host_row(b, l, c, h)


def test_single_page_direct_equals_layer_first():
    for L, C, ps in ((3, 2, 4), (4, 1, 8)):
        a = Geometry(L, C, 16, 8, ps, ps, PAGE_FIRST_DIRECT)
        b = a.replace(layout=LAYER_FIRST)
        for l in range(L):
            for c in range(C):
                for h in range(ps):
                    assert oracle.host_row(a, l, c, h) == oracle.host_row(b, l, c, h)


def test_contiguous_layer_first_is_a_slice_copy():
    rng = np.random.default_rng(11)
    g = Geometry(3, 2, 64, 100, 64, 16, LAYER_FIRST)
    dev, host = random_pool(rng, g)
    d0, h0, n = 17, 16, 40
    oracle_backup(g, dev, host, np.arange(d0, d0 + n), np.arange(h0, h0 + n))
    expect = np.full(g.host_bytes(), SENTINEL, np.uint8).reshape(g.L, g.C, g.S_host, g.R)
    expect[:, :, h0:h0 + n] = dev[:, :, d0:d0 + n]
    assert np.array_equal(host, expect.reshape(-1))


@pytest.mark.parametrize("layout", LAYOUTS)
def test_request_order_does_not_matter(layout):
    rng = np.random.default_rng(12)
    g = Geometry(3, 2, 32, 30, 24, 4, layout)
    dev, host_a = random_pool(rng, g)
    host_b = host_a.copy()
    d = rng.choice(g.S_dev, 15, replace=False)
    h = rng.choice(g.S_host, 15, replace=False)
    perm = rng.permutation(15)
    oracle_backup(g, dev, host_a, d, h)
    oracle_backup(g, dev, host_b, d[perm], h[perm])
    assert np.array_equal(host_a, host_b)


# ---- 6. brute force over every permutation of tiny requests -----------------------

def test_brute_force_tiny_pools():
    cases = 0
    for L, C, R, ps in itertools.product((1, 2), (1, 2), (16, 32), (1, 2, 4)):
        S = 4
        for layout in LAYOUTS:
            g = Geometry(L, C, R, 5, S, ps, layout)
            rng = np.random.default_rng(L * 100 + C * 10 + ps + layout * 1000 + R)
            dev = rng.integers(0, 256, size=(L, C, 5, R), dtype=np.uint8)
            src = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
            for n in (1, 2, 3):
                for hs in itertools.permutations(range(S), n):
                    ds = rng.choice(5, n, replace=False)
                    host = np.full(g.host_bytes(), SENTINEL, np.uint8)
                    host_np = host.copy()
                    assert oracle_backup(g, dev, host, ds, hs) == 0
                    np_ref.backup(dev, host_np, layout, L, C, S, ps, R, ds, hs)
                    assert np.array_equal(host, host_np)
                    rc, out = oracle_load(g, dev, src, ds, hs)
                    dev_np = dev.copy()
                    np_ref.load(dev_np, src, layout, L, C, S, ps, R, ds, hs)
                    assert rc == 0 and np.array_equal(out, dev_np)
                    # round trip back into the device layout
                    _, back = oracle_load(g, np.zeros_like(dev), host, ds, hs)
                    assert np.array_equal(back[:, :, ds], dev[:, :, ds])
                    cases += 1
    assert cases > 1000


# ---- 7. validation rules -------------------------------------------------------

def test_validation_codes():
    g = Geometry(4, 2, 32, 10, 8, 4, PAGE_FIRST)
    ok_d, ok_h = [1, 2, 3], [0, 5, 7]
    assert oracle.validate(g, 0, ok_d, ok_h, 0, 4) == oracle.OK
    assert oracle.validate(g, 0, [], [], 0, 4) == oracle.OK
    assert oracle.validate(g, 0, ok_d, ok_h, 2, 2) == oracle.OK       # empty layer range
    assert oracle.validate(g, 0, ok_d, ok_h, -1, 2) == oracle.EINVAL
    assert oracle.validate(g, 0, ok_d, ok_h, 3, 2) == oracle.EINVAL
    assert oracle.validate(g, 0, ok_d, ok_h, 0, 5) == oracle.EINVAL
    assert oracle.validate(g, 0, [10, 1, 2], ok_h, 0, 4) == oracle.ERANGE
    assert oracle.validate(g, 0, [-1, 1, 2], ok_h, 0, 4) == oracle.ERANGE
    assert oracle.validate(g, 0, ok_d, [0, 8, 1], 0, 4) == oracle.ERANGE
    # duplicates: destination is host for backup, device for load
    assert oracle.validate(g, 0, [1, 1, 2], ok_h, 0, 4) == oracle.OK
    assert oracle.validate(g, 1, [1, 1, 2], ok_h, 0, 4) == oracle.EDUP
    assert oracle.validate(g, 0, ok_d, [3, 4, 3], 0, 4) == oracle.EDUP
    assert oracle.validate(g, 1, ok_d, [3, 4, 3], 0, 4) == oracle.OK
    assert oracle.validate(g, 0, ok_d, [3, 4, 3], 0, 4, check_unique=False) == oracle.OK
    # a range error wins over a duplicate anywhere in the request
    assert oracle.validate(g, 0, [1, 2, 3, 4], [3, 3, 1, 9], 0, 4) == oracle.ERANGE
    # bad geometries
    for bad in (g.replace(R=24), g.replace(R=0), g.replace(S_host=10), g.replace(ps=0),
                g.replace(L=0), g.replace(layout=3), g.replace(S_dev=0)):
        assert oracle.check_geometry(bad) == oracle.EINVAL
        assert oracle.validate(bad, 0, ok_d, ok_h, 0, 1) == oracle.EINVAL


def test_failed_validation_modifies_nothing():
    rng = np.random.default_rng(13)
    g = Geometry(2, 2, 32, 10, 8, 4, LAYER_FIRST)
    dev, host = random_pool(rng, g)
    before = host.copy()
    assert oracle_backup(g, dev, host, [1, 2, 3], [0, 0, 1]) == oracle.EDUP
    assert oracle_backup(g, dev, host, [1, 2, 30], [0, 2, 1]) == oracle.ERANGE
    assert np.array_equal(host, before)
    rc, out = oracle_load(g, dev, host, [1, 1, 3], [0, 2, 1])
    assert rc == oracle.EDUP and np.array_equal(out, dev)
