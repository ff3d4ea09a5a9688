"""GPU parity at the full workload sizes, through the C ABI.

Each workload runs in the launch configuration bench.py times. Full pools are
too large to mirror on the host in every case, so the oracle computes sampled
outputs: whole layers on compacted mirrors (the device rows a request touches,
gathered by torch), or rows addressed one by one through the oracle's host-row
map. Properties that hold at any size are checked on every buffer: device rows
outside the request are untouched (sum over them unchanged), host slots outside
the request keep the sentinel.
"""
import threading

import numpy as np
import pytest

import hierarchical_kv_cache_backup_amd as kvt
from hierarchical_kv_cache_backup_amd import workloads
import oracle
from oracle import Geometry, np_ref

from gpu_util import SENTINEL, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    t = torch_mod()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


def make_bufs(torch, shape, cfg, S_dev):
    bufs = []
    for l in range(shape.layers):
        for c in range(shape.components):
            b = torch.empty(S_dev * shape.row_bytes, dtype=torch.uint8, device="cuda:0")
            workloads.fill_device_buffer(b, shape, cfg, l, c, torch)
            bufs.append(b)
    return bufs


def release(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def rows_of(torch, buf, R, idx):
    """Device rows `idx` of one buffer, as a host numpy array (n, R)."""
    t = torch.from_numpy(np.asarray(idx, dtype=np.int64)).cuda()
    return buf.view(-1, R).index_select(0, t).cpu().numpy()


def untouched_sum(torch, buf, R, idx):
    mask = torch.ones(buf.numel() // R, dtype=torch.bool, device=buf.device)
    mask[torch.from_numpy(np.asarray(idx, dtype=np.int64)).cuda()] = False
    return int(buf.view(-1, R)[mask].to(torch.int64).sum())


def check_backup_layers(torch, g, pool, bufs, dev_idx, host_idx, layers, samples=2048):
    """Host rows written by a backup, for the given layers: a sample of positions,
    each row addressed through the oracle's host-row map and compared with the
    device row it must hold."""
    n = len(dev_idx)
    host = pool.host_array()
    for l in layers:
        pick = np.random.default_rng(l).choice(n, size=min(n, samples), replace=False)
        for c in range(g.C):
            m = rows_of(torch, bufs[l * g.C + c], g.R, np.asarray(dev_idx)[pick])
            for j, i in enumerate(pick):
                r = oracle.host_row(g, l, c, int(host_idx[i]))
                assert np.array_equal(host[r * g.R:(r + 1) * g.R], m[j]), (l, c, int(i))


def fill_host_random(torch, pool, seed):
    """Seeded random bytes into the host pool, made on the device in 1 GiB pieces
    and copied through a CPU tensor aliasing the pinned pool."""
    host = torch.from_numpy(pool.host_array())
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    piece = 1 << 30
    for off in range(0, host.numel(), piece):
        m = min(piece, host.numel() - off)
        host[off:off + m].copy_(torch.empty(m, dtype=torch.uint8, device="cuda:0")
                                .random_(0, 256, generator=g))
    torch.cuda.synchronize()


def check_load_layers(torch, g, pool, bufs, dev_idx, host_idx, layers):
    """Device rows written by a load, for the given layers, against the oracle run
    on compacted mirrors reading the live host pool."""
    n = len(dev_idx)
    host = pool.host_array()
    gl = g.replace(S_dev=n)
    for l in layers:
        mirrors = [np.zeros(0, np.uint8)] * (g.L * g.C)
        for c in range(g.C):
            mirrors[l * g.C + c] = np.zeros(n * g.R, np.uint8)
        assert oracle.load(gl, mirrors, host, np.arange(n), host_idx, l, l + 1) == 0
        for c in range(g.C):
            got = rows_of(torch, bufs[l * g.C + c], g.R, dev_idx)
            want = mirrors[l * g.C + c].reshape(n, g.R)
            assert np.array_equal(got, want), (l, c)


def sample_layers(L):
    return sorted({0, L // 3, (2 * L) // 3, L - 1})


# ---- llama8b: D2H of an 8192-token prefix from fragmented pages ------------------

@pytest.mark.parametrize("path", (kvt.PATH_AUTO, kvt.PATH_KERNEL, "kernel_full_grid",
                                  kvt.PATH_KERNEL_LDS, kvt.PATH_DMA, kvt.PATH_STAGED))
def test_llama8b_fragmented_backup(torch, path):
    shape = workloads.llama8b()
    n = shape.extra["tokens"]
    bufs = make_bufs(torch, shape, 2, shape.device_slots)
    dev_idx, host_idx = workloads.prefix_indices(shape, 2, n, fragmented=True)
    for layout in shape.layouts:
        g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                     shape.host_slots, shape.page_size, layout)
        print("llama8b layout=%d path=%s n=%d" % (layout, path, n), flush=True)
        with kvt.KvPool(kvt.geometry(*g.args()), bufs) as pool:
            if path == "kernel_full_grid":        # the write-back kernel without its cap
                c = pool.calibration()
                c.kernel_max_workgroups[0] = 0
                pool.set_calibration(c)
                pool.set_path(kvt.PATH_KERNEL)
            else:
                pool.set_path(path)
            pool.host_array()[:] = SENTINEL
            s = torch.cuda.Stream()
            pool.backup(dev_idx, host_idx, 0, g.L, s)
            s.synchronize()
            # the whole host image: oracle on full compacted mirrors (8192 rows per buffer)
            mirrors = [rows_of(torch, b, g.R, dev_idx).reshape(-1) for b in bufs]
            want = np.full(g.host_bytes(), SENTINEL, np.uint8)
            assert oracle.backup(g.replace(S_dev=n), mirrors, want, np.arange(n), host_idx) == 0
            assert np.array_equal(pool.host_array(), want)
    del bufs
    release(torch)


# ---- mla32k: H2D of a 32768-token prefix, page_first_direct vs layer_first -------

@pytest.mark.parametrize("path", (kvt.PATH_AUTO, kvt.PATH_KERNEL, kvt.PATH_KERNEL_LDS, kvt.PATH_DMA,
                                  kvt.PATH_STAGED))
@pytest.mark.timeout(300)
def test_mla32k_load(torch, path):
    shape = workloads.mla32k()
    n = shape.extra["tokens"]
    bufs = make_bufs(torch, shape, 3, shape.device_slots)
    for fragmented in (False, True):
        dev_idx, host_idx = workloads.prefix_indices(shape, 3, n, fragmented=fragmented)
        before = [untouched_sum(torch, b, shape.row_bytes, dev_idx) for b in bufs]
        for layout in shape.layouts:
            g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                         shape.host_slots, shape.page_size, layout)
            print("mla32k layout=%d path=%d fragmented=%d" % (layout, path, fragmented), flush=True)
            with kvt.KvPool(kvt.geometry(*g.args()), bufs) as pool:
                pool.set_path(path)
                fill_host_random(torch, pool, 30 + layout)
                s = torch.cuda.Stream()
                pool.load(dev_idx, host_idx, 0, g.L, s)
                s.synchronize()
                layers = range(g.L) if path == kvt.PATH_KERNEL else sample_layers(g.L)
                check_load_layers(torch, g, pool, bufs, dev_idx, host_idx, layers)
            after = [untouched_sum(torch, b, shape.row_bytes, dev_idx) for b in bufs]
            assert after == before
    del bufs
    release(torch)


# ---- mixed batch: H2D of L2 hits concurrent with D2H of new pages ---------------------

# (write-back path, load path) pairings the mixed batch runs with; AUTO on a
# pool flagged KV_F_DUPLEX is the pairing bench.py times
MIXED_PAIRINGS = (("kernel", kvt.PATH_KERNEL, kvt.PATH_KERNEL),
                  ("auto_duplex", kvt.PATH_AUTO, kvt.PATH_AUTO),
                  ("staged", kvt.PATH_STAGED, kvt.PATH_STAGED),
                  ("dma", kvt.PATH_DMA, kvt.PATH_DMA),
                  ("staged_back_kernel_load", kvt.PATH_STAGED, kvt.PATH_KERNEL))


def reset_host_slots(g, pool, host_idx, value):
    """Sets the host rows of slots host_idx, every layer and component, to value,
    through the oracle's NumPy view of the host pool in the layout's own
    dimension order."""
    view = np_ref.host_view(pool.host_array(), g.layout, g.L, g.C, g.S_host, g.ps, g.R)
    key, _ = np_ref._host_rows(view, g.layout, host_idx, 0, g.L, g.ps)
    view[key] = value


@pytest.mark.timeout(1100)
def test_mixed_bidirectional(torch):
    """The mixed batch at full size (~54 GB each way in all): the L2 hits load
    while the new pages write back, from two threads on two library streams
    against one pool flagged KV_F_DUPLEX, on every pairing of MIXED_PAIRINGS,
    in both of its layouts. Before each pairing the hit rows on the device and
    the new pages' host rows are reset to the sentinel; afterwards sampled
    layers are compared with the oracle and every other device row is
    unchanged."""
    shape = workloads.mixed()
    plan = workloads.mixed_plan(shape, 4)
    S_dev, S_host = plan["device_slots"], plan["host_slots"]
    h_dev, h_host = plan["h2d"]
    w_dev, w_host = plan["d2h"]
    print("mixed: %d tokens, %d hits, %d new" % (S_dev, h_dev.size, w_dev.size), flush=True)
    bufs = make_bufs(torch, shape, 4, S_dev)
    both = np.concatenate([h_dev, w_dev])
    t_hits = torch.from_numpy(h_dev).cuda()
    for layout in shape.layouts:
        g = Geometry(shape.layers, shape.components, shape.row_bytes, S_dev, S_host,
                     shape.page_size, layout)
        with kvt.KvPool(kvt.geometry(*g.args()), bufs,
                        flags=kvt.F_CHECK_UNIQUE | kvt.F_DUPLEX) as pool:
            pool.set_path(kvt.PATH_KERNEL)
            s_load, s_back = kvt.Stream(), kvt.Stream()
            # L2 holds the hit pages: write them back once
            pool.backup(h_dev, h_host, 0, g.L, s_back)
            s_back.synchronize()
            untouched = [untouched_sum(torch, b, g.R, both) for b in bufs]
            for name, back_path, load_path in MIXED_PAIRINGS:
                print("mixed layout=%d pairing=%s" % (layout, name), flush=True)
                reset_host_slots(g, pool, w_host, SENTINEL)
                for b in bufs:
                    b.view(-1, g.R)[t_hits] = SENTINEL
                torch.cuda.synchronize()
                pool.set_path(back_path, kvt.BACKUP)
                pool.set_path(load_path, kvt.LOAD)
                go = threading.Barrier(2)
                errors = []

                def run(fn):
                    try:
                        go.wait()
                        fn()
                    except Exception as e:  # surfaced below
                        errors.append(e)

                th = [threading.Thread(target=run, args=(
                          lambda: pool.load(h_dev, h_host, 0, g.L, s_load),)),
                      threading.Thread(target=run, args=(
                          lambda: pool.backup(w_dev, w_host, 0, g.L, s_back),))]
                for x in th:
                    x.start()
                for x in th:
                    x.join()
                assert not errors, errors
                s_load.synchronize()
                s_back.synchronize()
                used = (kvt.PATH_NAMES[pool.last_path(kvt.BACKUP)],
                        kvt.PATH_NAMES[pool.last_path(kvt.LOAD)])
                print("mixed layout=%d pairing=%s ran backup=%s load=%s" % ((layout, name) + used),
                      flush=True)
                layers = sample_layers(g.L)
                check_load_layers(torch, g, pool, bufs, h_dev, h_host, layers)
                check_backup_layers(torch, g, pool, bufs, w_dev, w_host, layers)
                assert [untouched_sum(torch, b, g.R, both) for b in bufs] == untouched
            s_load.close()
            s_back.close()
    del bufs
    release(torch)


# ---- streamed: per-layer H2D overlapped with a consumer on another stream ---------------

@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant", ("kernel", "dma", "staged", "auto_overlap"))
def test_streamed_per_layer_events(torch, variant):
    """The 61-layer fp8 prefix (256 MiB per layer) loads while a consumer on
    another stream sums each layer right after kv_load_layer(l), on the kernel,
    copy-engine and staged paths and on AUTO with KV_F_LOAD_OVERLAP; every
    layer's sum and sampled layers' bytes match."""
    path, flags = {"kernel": (kvt.PATH_KERNEL, kvt.F_CHECK_UNIQUE),
                   "dma": (kvt.PATH_DMA, kvt.F_CHECK_UNIQUE),
                   "staged": (kvt.PATH_STAGED, kvt.F_CHECK_UNIQUE),
                   "auto_overlap": (kvt.PATH_AUTO,
                                    kvt.F_CHECK_UNIQUE | kvt.F_LOAD_OVERLAP)}[variant]
    shape = workloads.streamed()
    n = shape.extra["tokens"]
    bufs = make_bufs(torch, shape, 5, shape.device_slots)
    dev_idx, host_idx = workloads.prefix_indices(shape, 5, n, fragmented=False)
    t_idx = torch.from_numpy(dev_idx).cuda()
    for layout in shape.layouts:
        g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                     shape.host_slots, shape.page_size, layout)
        print("streamed %s layout=%d" % (variant, layout), flush=True)
        with kvt.KvPool(kvt.geometry(*g.args()), bufs, flags=flags) as pool:
            pool.set_path(kvt.PATH_KERNEL)
            s_load, s_comp = torch.cuda.Stream(), torch.cuda.Stream()
            # L2 content: written back from the device pool, then the device rows are cleared
            pool.backup(dev_idx, host_idx, 0, g.L, s_load)
            s_load.synchronize()
            pool.set_path(path)
            for b in bufs:
                b.view(-1, g.R)[t_idx] = 0
            torch.cuda.synchronize()
            pool.load(dev_idx, host_idx, 0, g.L, s_load)
            with torch.cuda.stream(s_comp):
                # made on the consumer's stream: a tensor filled on the default
                # stream and written here would race with that fill
                sums = torch.zeros(g.L * g.C, dtype=torch.int64, device="cuda:0")
                for l in range(g.L):
                    pool.load_layer(l, s_comp)
                    for c in range(g.C):
                        rows = bufs[l * g.C + c].view(-1, g.R).index_select(0, t_idx)
                        sums[l * g.C + c] = rows.to(torch.int64).sum()
            s_comp.synchronize()
            s_load.synchronize()
            for l in range(g.L):
                for c in range(g.C):
                    rows = bufs[l * g.C + c].view(-1, g.R).index_select(0, t_idx)
                    assert int(sums[l * g.C + c]) == int(rows.to(torch.int64).sum()), (l, c)
            check_load_layers(torch, g, pool, bufs, dev_idx, host_idx, sample_layers(g.L))
    del bufs
    release(torch)


# ---- mla32k with a host pool shared by a tensor-parallel group of two ---------------

@pytest.mark.timeout(300)
def test_mla32k_shared_host_pool(torch):
    """The 32768-token MLA prefix in a group of two pools sharing one host pool:
    the writer backs up (fragmented device pages), the other rank's backup moves
    nothing, and the other rank loads into its own device pool at other slots,
    on a second stream, with no host synchronisation after the writer's call."""
    shape = workloads.mla32k()
    n = shape.extra["tokens"]
    src = make_bufs(torch, shape, 3, shape.device_slots)
    dst = [torch.empty_like(b) for b in src]
    for b in dst:
        b.fill_(SENTINEL)
    dev_w, host_idx = workloads.prefix_indices(shape, 3, n, fragmented=True)
    dev_r, _ = workloads.prefix_indices(shape, 5, n, fragmented=True)
    g = Geometry(shape.layers, shape.components, shape.row_bytes, shape.device_slots,
                 shape.host_slots, shape.page_size, oracle.PAGE_FIRST_DIRECT)
    before = [untouched_sum(torch, b, shape.row_bytes, dev_r) for b in dst]
    writer = kvt.KvPool(kvt.geometry(*g.args()), src,
                        flags=kvt.F_CHECK_UNIQUE | kvt.F_SHARE_CHECK)
    reader = kvt.KvPool(kvt.geometry(*g.args()), dst, share_with=writer)
    s_w, s_r = torch.cuda.Stream(), torch.cuda.Stream()
    print("mla32k shared: writer backup, reader backup + load", flush=True)
    writer.backup(dev_w, host_idx, 0, g.L, s_w)
    reader.backup(dev_r, host_idx, 0, g.L, s_r)
    reader.load(dev_r, host_idx, 0, g.L, s_r)
    s_r.synchronize()
    s_w.synchronize()
    assert reader.last_path(kvt.BACKUP) == kvt.PATH_SHARED
    check_backup_layers(torch, g, writer, src, dev_w, host_idx, sample_layers(g.L))
    check_load_layers(torch, g, reader, dst, dev_r, host_idx, range(g.L))
    for l in range(g.L):        # every row the reader holds is the writer's source row
        a = src[l].view(-1, g.R).index_select(0, torch.from_numpy(dev_w).cuda())
        b = dst[l].view(-1, g.R).index_select(0, torch.from_numpy(dev_r).cuda())
        assert torch.equal(a, b), l
    after = [untouched_sum(torch, b, shape.row_bytes, dev_r) for b in dst]
    assert after == before
    reader.close()
    writer.close()
    del src, dst
    release(torch)


# ---- kv_load_layer gating at full size, on every path and kind of load stream --------

@pytest.mark.timeout(300)
@pytest.mark.parametrize("stream_kind", ("torch", "library"))
@pytest.mark.parametrize("path", (kvt.PATH_KERNEL, kvt.PATH_DMA, kvt.PATH_STAGED))
def test_load_layer_gates_consumer_at_full_size(torch, path, stream_kind):
    """The MLA prefix (16384 and 32768 tokens, one landed event per layer) loads
    on a torch stream or on a library stream (kv_stream_create); a consumer on
    another stream reads each layer right after kv_load_layer(l) and must see the
    loaded bytes in every layer, on the kernel, copy-engine and staged paths (the
    staged path records its landed events on its own auxiliary stream). A wait
    that does not hold shows as a layer read before it landed."""
    shape = workloads.mla32k()
    L, R, S_dev = shape.layers, shape.row_bytes, shape.device_slots
    bufs = make_bufs(torch, shape, 3, S_dev)
    g = Geometry(L, 1, R, S_dev, shape.host_slots, shape.page_size, oracle.LAYER_FIRST)
    pool = kvt.KvPool(kvt.geometry(*g.args()), bufs)
    lib_stream = kvt.Stream() if stream_kind == "library" else None
    s = lib_stream.torch if lib_stream else torch.cuda.Stream()
    c = torch.cuda.Stream()
    for n in (16384, 32768):
        src = np.arange(n, dtype=np.int64)
        dst = src + (S_dev - n)
        host = np.arange(n, dtype=np.int64)
        pool.set_path(kvt.PATH_KERNEL)
        pool.backup(src, host, 0, L, s)
        s.synchronize()
        pool.set_path(path)
        want = torch.stack([bufs[l].view(S_dev, R)[:n].to(torch.int64).sum() for l in range(L)])
        for rep in range(3):
            for l in range(L):
                bufs[l].view(S_dev, R)[S_dev - n:].zero_()
            torch.cuda.synchronize()
            print("gating path=%d stream=%s n=%d rep=%d" % (path, stream_kind, n, rep), flush=True)
            pool.load(dst, host, 0, L, s)
            with torch.cuda.stream(c):
                sums = torch.zeros(L, dtype=torch.int64, device="cuda:0")
                for l in range(L):
                    pool.load_layer(l, c)
                    sums[l] = bufs[l].view(S_dev, R)[S_dev - n:].to(torch.int64).sum()
            c.synchronize()
            s.synchronize()
            early = [l for l in range(L) if int(sums[l]) != int(want[l])]
            assert not early, ("layers read before they landed", early[:10], len(early))
            for l in sample_layers(L):
                assert torch.equal(bufs[l].view(S_dev, R)[S_dev - n:], bufs[l].view(S_dev, R)[:n])
    pool.close()
    if lib_stream:
        lib_stream.close()
    del bufs
    release(torch)
