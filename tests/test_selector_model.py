"""The path selector's time model on the host (kv_model_path, no GPU).

The model prices a request on the kernel, copy-engine and staged paths:

* the formulas as include/kvtier.h documents them, on synthetic calibrations;
* the flags (overlap, duplex) and the argument checks;
* the default calibration against measured outcomes. AUTO's choice is checked
  against the path that was fastest on an MI355X in `bench.py --size-sweep`
  (78 x 1152 B MLA latent, contiguous slots; measured GB/s in the comments).
"""
import math

import numpy as np
import pytest

kvt = pytest.importorskip("hierarchical_kv_cache_backup_amd")

MLA = dict(L=78, C=1, R=1152, S_dev=65536, S_host=32768, ps=64)
LAYOUT = {"layer_first": 0, "page_first": 1, "page_first_direct": 2}


def _geom(layout, **kw):
    p = dict(MLA, **kw)
    return kvt.geometry(p["L"], p["C"], p["R"], p["S_dev"], p["S_host"], p["ps"], layout)


def _default():
    rc, c = kvt.kv_default_calibration()
    assert rc == kvt.OK
    return c


def _req(n):
    return np.arange(n, dtype=np.int64) + 128, np.arange(n, dtype=np.int64)


def test_closed_form_uncapped_and_capped_kernel():
    """kernel = launch + (groups-1) x (gap + link gap) + max(bytes/rate,
    capped-grid term); copy engines = copies x per-copy cost + bytes/rate."""
    g = kvt.geometry(4, 2, 4096, 4096, 4096, 16, 0)
    c = _default()
    c.kernel_launch_us[:] = [20.0, 20.0]
    c.kernel_group_us[:] = [5.0, 5.0]
    c.kernel_link_gap_us[:] = [0.0, 3.0]
    c.kernel_gbps[:] = [50.0, 40.0]
    c.dma_copy_us[:] = [10.0, 10.0]
    c.dma_gbps[:] = [25.0, 20.0]
    c.load_split_min_bytes = 1.0              # one group per layer
    c.kernel_max_workgroups[:] = [0, 0]
    c.kernel_wg_jump_ns[:] = [0.0, 0.0]
    d, h = _req(1024)
    nbytes = 1024 * 4 * 2 * 4096
    rc, t = kvt.kv_model_path(g, c, 1, d, h, 0, 4)
    assert rc >= 0
    assert t[0] == pytest.approx(20 + 3 * (5 + 3) + nbytes / 40e3)
    # contiguous on both sides: one copy per (layer, component)
    assert t[1] == pytest.approx(8 * 10 + nbytes / 20e3)
    # capped write-back: 24 workgroups of 2 GB/s, 100 ns per row, a 50 us
    # start over the first 16 MiB (the 32 MiB call pays all of it)
    c.kernel_max_workgroups[:] = [24, 0]
    c.kernel_wg_gbps[:] = [2.0, 2.0]
    c.kernel_wg_row_ns[:] = [100.0, 0.0]
    c.kernel_wg_start_bytes[:] = [16 * 2 ** 20, 0]
    c.kernel_wg_start_us[:] = [50.0, 0.0]
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
    rows = 1024 * 8
    t_wg = (rows * 100e-3 + nbytes / 2e3) / 24          # before the slow start
    assert t[0] == pytest.approx(20 + max(nbytes / 50e3, t_wg) + 50.0)
    # a cap above the block count leaves the grid whole (4 rows of 4 KiB per
    # 16 KiB block: 2048 blocks) and takes no slow start
    c.kernel_max_workgroups[:] = [4096, 0]
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
    assert t[0] == pytest.approx(20 + max(nbytes / 50e3, (rows * 100e-3 + nbytes / 2e3) / 2048))
    # a paced capped grid moves no faster than its pace past each workgroup's
    # burst (24 x 16 blocks of 4 rows of 4 KiB), and the slow start comes on
    # top of whichever bound holds; the pace does not apply to a grid of one
    # workgroup per block, and 0 is unpaced
    c.kernel_max_workgroups[:] = [24, 0]
    burst_bytes = 24 * 16 * 4 * 4096
    yld = 0.99                                          # what a paced grid delivers
    for pace, burst, want in ((10.0, 0, nbytes / (yld * 10e3)),
                              (10.0, 16, (nbytes - burst_bytes) / (yld * 10e3)),
                              (1000.0, 0, t_wg), (0.0, 16, t_wg)):
        c.kernel_pace_gbps[:] = [pace, 0.0]
        c.kernel_pace_burst_blocks[:] = [burst, 0.0]
        rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
        assert t[0] == pytest.approx(20 + max(nbytes / 50e3, t_wg, want) + 50.0), (pace, burst)
    c.kernel_pace_burst_blocks[:] = [10 ** 4, 0.0]     # a burst past the call: unpaced
    c.kernel_pace_gbps[:] = [10.0, 0.0]
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
    assert t[0] == pytest.approx(20 + max(nbytes / 50e3, t_wg) + 50.0)
    # jumps: walk rows whose device row does not follow the previous walk row's,
    # (layers x C) x the runs of consecutive device slots in each walk group:
    # contiguous slots make one run in layer_first, one per position in
    # page_first and one per 16-token page in page_first_direct; reversed
    # slots make one per position everywhere
    c.kernel_pace_gbps[:] = [0.0, 0.0]
    c.kernel_wg_row_ns[:] = [0.0, 0.0]
    c.kernel_wg_jump_ns[:] = [50.0, 0.0]
    for layout, slots, runs in ((0, d, 1), (1, d, 1024), (2, d, 1024 // 16),
                                (0, d[::-1].copy(), 1024), (2, d[::-1].copy(), 1024)):
        g2 = kvt.geometry(4, 2, 4096, 4096, 4096, 16, layout)
        rc, t = kvt.kv_model_path(g2, c, 0, slots, h, 0, 4)
        want_wg = (runs * 8 * 50e-3 + nbytes / 2e3) / 24 + 50.0
        assert t[0] == pytest.approx(20 + max(nbytes / 50e3, want_wg)), (layout, runs)
    c.kernel_max_workgroups[:] = [4096, 0]
    c.kernel_pace_gbps[:] = [10.0, 0.0]
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
    assert t[0] == pytest.approx(20 + max(nbytes / 50e3, (rows * 100e-3 + nbytes / 2e3) / 2048))
    for bad in (0.5, -1.0, float("nan")):
        c.kernel_pace_gbps[:] = [bad, 0.0]
        rc, _ = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
        assert rc == kvt.EINVAL, bad
    c.kernel_pace_gbps[:] = [10.0, 0.0]
    for bad in (0.5, -1.0, 65537.0, float("nan")):
        c.kernel_pace_burst_blocks[:] = [bad, 0.0]
        rc, _ = kvt.kv_model_path(g, c, 0, d, h, 0, 4)
        assert rc == kvt.EINVAL, bad
    c.kernel_pace_burst_blocks[:] = [0.0, 0.0]
    c.kernel_wg_jump_ns[:] = [-1.0, 0.0]
    assert kvt.kv_model_path(g, c, 0, d, h, 0, 4)[0] == kvt.EINVAL


def test_staged_closed_form_with_and_without_ramp():
    """staged = (extents + ramp) x per-copy cost + launch + (chunks-1) x gap
    + bytes/copy rate + the one exposed device pass: half/64 on a ramped
    unit, else the whole half."""
    g = _geom(LAYOUT["page_first"])
    c = _default()
    d, h = _req(4096)                     # one host extent in page_first
    nbytes = 4096 * 78 * 1152
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 78)
    half = min(c.staged_chunk_bytes, nbytes)
    chunks = math.ceil(nbytes / c.staged_chunk_bytes) + 1 + 2
    want = ((1 + 2) * c.dma_copy_us[0] + c.kernel_launch_us[0] + (chunks - 1) * c.kernel_group_us[0]
            + nbytes / (c.dma_gbps[0] * 1e3) + half / 64 / (c.staged_gather_gbps * 1e3))
    assert t[2] == pytest.approx(want)
    # a half below staged_chunk_bytes / 16 does not ramp: the whole pass shows
    d, h = _req(64)
    nbytes = 64 * 78 * 1152
    rc, t = kvt.kv_model_path(g, c, 0, d, h, 0, 78)
    want = (1 * c.dma_copy_us[0] + c.kernel_launch_us[0] + 1 * c.kernel_group_us[0]
            + nbytes / (c.dma_gbps[0] * 1e3) + nbytes / (c.staged_gather_gbps * 1e3))
    assert t[2] == pytest.approx(want)


def test_flags_overlap_and_duplex():
    c = _default()
    d, h = _req(4096)
    for name, lay in LAYOUT.items():
        g = _geom(lay)
        p0, t0 = kvt.kv_model_path(g, c, 1, d, h, 0, 78)
        p1, t1 = kvt.kv_model_path(g, c, 1, d, h, 0, 78, kvt.F_LOAD_OVERLAP)
        assert t1[0] == pytest.approx(t0[0] * (1 + c.overlap_kernel_penalty))
        assert t1[1] == pytest.approx(t0[1] * (1 + c.overlap_dma_penalty))
        if name == "layer_first":
            assert t1[2] == pytest.approx(t0[2] * (1 + c.overlap_dma_penalty))
        else:   # one unit: every layer would land at the end of the load
            assert math.isinf(t1[2]) and p1 != kvt.PATH_STAGED
        # duplex: the kernel path is charged its penalty and runs on the
        # smaller of the two grid caps (the duplex cap, 24, below the default 26)
        p2, t2 = kvt.kv_model_path(g, c, 0, d, h, 0, 78, kvt.F_DUPLEX)
        p3, t3 = kvt.kv_model_path(g, c, 0, d, h, 0, 78)
        c24 = _default()
        assert c.duplex_kernel_max_workgroups[0] < c.kernel_max_workgroups[0]
        c24.kernel_max_workgroups[0] = c.duplex_kernel_max_workgroups[0]
        p5, t5 = kvt.kv_model_path(g, c24, 0, d, h, 0, 78)
        assert t2[0] == pytest.approx(t5[0] * (1 + c.duplex_kernel_penalty[0]))
        assert t2[0] > t3[0] * (1 + c.duplex_kernel_penalty[0])
        assert t2[1] == t3[1] and t2[2] == t3[2]
        # backups never take the overlap charge
        p4, t4 = kvt.kv_model_path(g, c, 0, d, h, 0, 78, kvt.F_LOAD_OVERLAP)
        assert t4 == t3


# (layout, tokens, direction) -> path AUTO must take with the default
# calibration; in brackets the GB/s measured per path (kernel / copy engines /
# staged) by bench.py --size-sweep on an MI355X.
MEASURED = [
    ("layer_first", 256, 0, kvt.PATH_KERNEL),          # 33.1 / 19.8 / 19.0
    ("layer_first", 2048, 0, kvt.PATH_KERNEL),         # 49.4 / 46.1 / 45.5
    ("page_first", 256, 0, kvt.PATH_STAGED),           # 31.9 / 19.8 / 44.5
    ("page_first", 1024, 0, kvt.PATH_STAGED),          # 45.4 / 38.1 / 53.1
    ("page_first", 8192, 0, kvt.PATH_STAGED),          # 52.7 / 53.1 / 56.2
    ("page_first", 16384, 0, kvt.PATH_STAGED),         # 53.2 / 54.8 / 56.3
    ("page_first_direct", 256, 0, kvt.PATH_STAGED),    # 32.7 / 19.6 / 44.8
    ("page_first_direct", 4096, 0, kvt.PATH_STAGED),   # 51.5 / 50.5 / 55.6
    ("layer_first", 1024, 1, kvt.PATH_KERNEL),         # 55.1 / 38.3 / 36.5
    ("layer_first", 8192, 1, kvt.PATH_KERNEL),         # 56.0 / 53.2 / 50.4
    ("page_first", 256, 1, kvt.PATH_KERNEL),           # 51.9 / 20.0 / 45.4
    ("page_first_direct", 512, 1, kvt.PATH_KERNEL),    # 54.5 / 29.6 / 50.6
]


@pytest.mark.parametrize("layout,tokens,direction,want", MEASURED)
def test_default_model_picks_the_measured_best_path(layout, tokens, direction, want):
    d, h = _req(tokens)
    path, t = kvt.kv_model_path(_geom(LAYOUT[layout]), _default(), direction, d, h, 0, 78)
    assert path == want, (kvt.PATH_NAMES.get(path, path), [round(x) for x in t])


def test_argument_errors():
    c = _default()
    g = _geom(0)
    d, h = _req(16)
    assert kvt.kv_model_path(g, c, 2, d, h, 0, 78)[0] == kvt.EINVAL
    assert kvt.kv_model_path(g, c, 0, d[:0], h[:0], 0, 78)[0] == kvt.EINVAL     # empty
    assert kvt.kv_model_path(g, c, 0, d, h, 5, 5)[0] == kvt.EINVAL               # no layers
    bad = np.array(h)
    bad[3] = MLA["S_host"]
    assert kvt.kv_model_path(g, c, 0, d, bad, 0, 78)[0] == kvt.ERANGE
    c.dma_gbps[0] = 0.0
    assert kvt.kv_model_path(g, c, 0, d, h, 0, 78)[0] == kvt.EINVAL
    assert kvt.kv_default_calibration()[0] == kvt.OK
