"""kv_stage, the staged path's device-side pass on its own ("Baidu's KVCache
Overhaul", "DMA Segment Explosion & Batched Gather/Scatter"), through the C ABI.

The order of the rows in the staging buffer is derived from the oracle's NumPy
row-id table (the host pool's rows enumerated in storage order and viewed in
the layout's dimension order, no address formula): the request's positions
are taken as host slots 0..n-1 of a pool holding the requested layers, and the
rows are packed in increasing host row. Where the request fills whole pages,
the packed buffer must also equal the host image the C oracle's backup writes
for host slots 0..n-1.
"""
import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
from hierarchical_kv_cache_backup_amd import workloads
import oracle
from oracle import Geometry, np_ref

from gpu_util import device_buffers, kv_geom, mirrors, torch_mod

pytestmark = pytest.mark.gpu

LAYOUTS = (oracle.LAYER_FIRST, oracle.PAGE_FIRST, oracle.PAGE_FIRST_DIRECT)


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def stage_order(g, n, l0, l1):
    """(position, layer, comp) of each row of the staging buffer, in order."""
    Lp, C, ps = l1 - l0, g.C, g.ps
    S = -(-n // ps) * ps
    table = np_ref.row_id_table(g.layout, Lp, C, S, ps)[:, :, :n]     # (Lp, C, n) host rows
    order = np.argsort(table.reshape(-1), kind="stable")
    return order % n, order // (C * n) + l0, (order // n) % C


def expected_pack(g, dev_m, dev_idx, l0, l1):
    i, l, c = stage_order(g, len(dev_idx), l0, l1)
    out = np.empty((i.size, g.R), np.uint8)
    for k in range(i.size):
        d = int(dev_idx[i[k]])
        out[k] = dev_m[l[k] * g.C + c[k]][d * g.R:(d + 1) * g.R]
    return out.reshape(-1)


CASES = [  # (L, C, R, S_dev, ps, n, l0, l1)
    (4, 2, 272, 700, 16, 512, 0, 4),     # whole pages
    (4, 2, 272, 700, 16, 437, 1, 3),     # ragged last page, a layer sub-range
    (3, 1, 1152, 300, 64, 200, 0, 3),
    (2, 2, 48, 900, 1, 777, 0, 2),
    (5, 1, 16, 2000, 4, 1999, 2, 5),
    (2, 2, 4096, 64, 8, 40, 0, 2),       # rows larger than a wave's pass
    (3, 2, 512, 600, 16, 333, 0, 3),     # half a window: two whole rows per window
    (2, 1, 1024, 500, 8, 257, 0, 2),     # exactly one window per row
    (2, 2, 1040, 300, 4, 123, 1, 2),     # the narrowest rows that straddle windows
    (2, 1, 1008, 300, 4, 201, 0, 2),     # the widest rows shorter than a window
]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_stage_pack_and_unpack_match_oracle(torch, layout, case):
    L, C, R, S_dev, ps, n, l0, l1 = CASES[case]
    S_host = -(-S_dev // ps) * ps
    g = Geometry(L, C, R, S_dev, S_host, ps, layout)
    print("stage case=%d layout=%d" % (case, layout), flush=True)
    rng = np.random.default_rng(100 + case)
    dev_idx = rng.choice(S_dev, n, replace=False).astype(np.int64)
    bufs = device_buffers(g, seed=110 + case)
    pool = kvt.KvPool(kv_geom(g), bufs)
    s = torch.cuda.Stream()
    rows = n * (l1 - l0) * C
    stage = torch.full((rows * R,), 0x5A, dtype=torch.uint8, device="cuda:0")
    dev_m = mirrors(bufs)
    pool.stage(0, dev_idx, stage, l0, l1, s)
    s.synchronize()
    want = expected_pack(g, dev_m, dev_idx, l0, l1)
    assert np.array_equal(stage.cpu().numpy(), want)
    if n % ps == 0:   # whole pages: the packed rows are the host image of slots 0..n-1
        gs = g.replace(L=l1 - l0, S_host=n)
        host = np.zeros(gs.host_bytes(), np.uint8)
        sub = dev_m[l0 * C:l1 * C]
        assert oracle.backup(gs, sub, host, dev_idx, np.arange(n)) == 0
        assert np.array_equal(want, host)
    # unpack random bytes into the same slots: those rows take the stage's
    # bytes, every other byte of the device pool is unchanged
    src = rng.integers(0, 256, rows * R, dtype=np.uint8)
    stage.copy_(torch.from_numpy(src))
    torch.cuda.synchronize()
    pool.stage(1, dev_idx, stage, l0, l1, s)
    s.synchronize()
    i, l, c = stage_order(g, n, l0, l1)
    for k in range(i.size):
        d = int(dev_idx[i[k]])
        dev_m[l[k] * C + c[k]][d * R:(d + 1) * R] = src[k * R:(k + 1) * R]
    for k, b in enumerate(bufs):
        assert np.array_equal(b.cpu().numpy(), dev_m[k]), k
    pool.close()


def test_stage_errors(torch):
    g = Geometry(2, 1, 64, 64, 64, 8, 0)
    bufs = device_buffers(g, seed=5)
    pool = kvt.KvPool(kv_geom(g), bufs)
    h = pool.handle
    stage = torch.zeros(16 * 2 * 64 + 16, dtype=torch.uint8, device="cuda:0")
    idx = np.arange(16)
    p = stage.data_ptr()
    assert kvt.kv_stage(h, 0, idx, 0, 2, p) == kvt.OK
    assert kvt.kv_stage(h, 2, idx, 0, 2, p) == kvt.EINVAL
    assert kvt.kv_stage(h, 0, idx, 0, 3, p) == kvt.EINVAL
    assert kvt.kv_stage(h, 0, idx, 0, 2, None) == kvt.EINVAL
    assert kvt.kv_stage(h, 0, idx, 0, 2, p + 8) == kvt.EINVAL          # misaligned
    assert kvt.kv_stage(h, 0, [70], 0, 2, p) == kvt.ERANGE
    assert kvt.kv_stage(h, 1, [3, 3], 0, 2, p) == kvt.EDUP
    assert kvt.kv_stage(h, 0, [3, 3], 0, 2, p) == kvt.OK               # a pack may repeat
    host = torch.zeros(16 * 2 * 64, dtype=torch.uint8, pin_memory=True)
    assert kvt.kv_stage(h, 0, idx, 0, 2, host.data_ptr()) == kvt.EINVAL
    assert kvt.kv_stage(h, 0, idx, 0, 2, p, n=0) == kvt.OK
    torch.cuda.synchronize()
    pool.close()
    # a stage smaller than the request, past the end of the device allocation
    # that holds it (the library sees allocations, not tensors carved from them)
    g = Geometry(2, 1, 64, 1 << 20, 64, 8, 0)
    bufs = device_buffers(g, seed=6, fill=0)
    pool = kvt.KvPool(kv_geom(g), bufs)
    small = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    assert kvt.kv_stage(pool.handle, 0, np.arange(1 << 19), 0, 2, small.data_ptr()) == kvt.EINVAL
    pool.close()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("layout", (oracle.LAYER_FIRST, oracle.PAGE_FIRST_DIRECT))
def test_stage_full_prefix(torch, layout):
    """The 32768-token MLA prefix, all 78 layers, in one pack (2.94 GB, the
    launch bench.py times) from fragmented device pages, then unpacked into
    other slots: sampled stage rows against the oracle's order, and the
    unpacked rows equal the packed ones in every layer."""
    shape = workloads.mla32k()
    n, L, R = shape.extra["tokens"], shape.layers, shape.row_bytes
    g = Geometry(L, 1, R, shape.device_slots, shape.host_slots, shape.page_size, layout)
    bufs = []
    for l in range(L):
        b = torch.empty(g.S_dev * R, dtype=torch.uint8, device="cuda:0")
        workloads.fill_device_buffer(b, shape, 3, l, 0, torch)
        bufs.append(b)
    dev_idx, _ = workloads.prefix_indices(shape, 3, n, fragmented=True)
    pool = kvt.KvPool(kv_geom(g), bufs)
    s = torch.cuda.Stream()
    stage = torch.empty(n * L * R, dtype=torch.uint8, device="cuda:0")
    print("stage full prefix layout=%d" % layout, flush=True)
    pool.stage(0, dev_idx, stage, 0, L, s)
    s.synchronize()
    i, l, _ = stage_order(g, n, 0, L)
    pick = np.random.default_rng(7).choice(i.size, 4096, replace=False)
    st = stage.view(-1, R)
    for k in pick:
        row = bufs[l[k]].view(-1, R)[int(dev_idx[i[k]])]
        assert torch.equal(st[int(k)], row), int(k)
    ps = g.ps       # unpack into the pages the pack did not read, in random order
    free = np.setdiff1d(np.arange(g.S_dev // ps), np.unique(dev_idx // ps))
    other = workloads.page_indices(np.random.default_rng(8).permutation(free)[:n // ps], ps)
    pool.stage(1, other, stage, 0, L, s)
    s.synchronize()
    a, b = torch.from_numpy(dev_idx).cuda(), torch.from_numpy(other).cuda()
    for ll in range(L):
        assert torch.equal(bufs[ll].view(-1, R).index_select(0, a),
                           bufs[ll].view(-1, R).index_select(0, b)), ll
    pool.close()
    del bufs, stage
    torch.cuda.empty_cache()
