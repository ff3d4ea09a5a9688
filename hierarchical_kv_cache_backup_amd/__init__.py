"""Cross-tier KV transfer between a device KV pool and a pinned host KV pool.

Thin ctypes binding of libkvtier.so (C ABI declared in include/kvtier.h): the
functions below carry the C names and only marshal arguments; every step of a
transfer runs inside the library (host-side planning in C++, data movement in
gfx950 kernels or on the copy engines). PyTorch supplies device memory and
streams only.

The library must be built (``__graft_entry__.build()`` or
``python hierarchical_kv_cache_backup_amd/_build.py``); importing the binding
without it raises, there is no fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvtier.so")

OK, EINVAL, ERANGE, EDUP, ENOMEM, EHIP = 0, -1, -2, -3, -4, -5
ERROR_NAMES = {EINVAL: "KV_EINVAL", ERANGE: "KV_ERANGE", EDUP: "KV_EDUP",
               ENOMEM: "KV_ENOMEM", EHIP: "KV_EHIP"}
LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT = 0, 1, 2
PATH_AUTO, PATH_KERNEL, PATH_KERNEL_LDS, PATH_DMA, PATH_STAGED, PATH_SHARED = 0, 1, 2, 3, 4, 5
PATH_NAMES = {PATH_AUTO: "auto", PATH_KERNEL: "kernel", PATH_KERNEL_LDS: "kernel_lds",
              PATH_DMA: "dma", PATH_STAGED: "staged", PATH_SHARED: "shared", -1: "none"}
F_CHECK_UNIQUE, F_HOST_NONCOHERENT, F_LOAD_OVERLAP, F_DUPLEX, F_SHARE_CHECK = (
    0x1, 0x2, 0x4, 0x8, 0x10)
F_HOST_INTERLEAVE = 0x20
BACKUP, LOAD = 0, 1
FREE_FIFO, FREE_LIFO = 0, 1


class kv_geometry_t(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_components", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("device_slots", ctypes.c_int64),
                ("host_slots", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("host_layout", ctypes.c_int32)]


class kv_pool_desc_t(ctypes.Structure):
    _fields_ = [("geom", kv_geometry_t), ("device_buffers", ctypes.POINTER(ctypes.c_void_p)),
                ("device", ctypes.c_int32), ("numa_node", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class kv_calib_t(ctypes.Structure):
    _fields_ = [("kernel_launch_us", ctypes.c_double * 2), ("kernel_gbps", ctypes.c_double * 2),
                ("dma_copy_us", ctypes.c_double * 2), ("dma_gbps", ctypes.c_double * 2),
                ("load_split_min_bytes", ctypes.c_double),
                ("kernel_max_workgroups", ctypes.c_double * 2),
                ("overlap_kernel_penalty", ctypes.c_double),
                ("overlap_dma_penalty", ctypes.c_double),
                ("overlap_kernel_max_workgroups", ctypes.c_double),
                ("duplex_kernel_penalty", ctypes.c_double * 2),
                ("staged_chunk_bytes", ctypes.c_double),
                ("staged_gather_gbps", ctypes.c_double),
                ("kernel_group_us", ctypes.c_double * 2),
                ("staged_min_gain", ctypes.c_double),
                ("index_zero_copy_max_bytes", ctypes.c_double * 2),
                ("duplex_kernel_max_workgroups", ctypes.c_double * 2),
                ("kernel_wg_gbps", ctypes.c_double * 2),
                ("kernel_wg_row_ns", ctypes.c_double * 2),
                ("kernel_wg_start_bytes", ctypes.c_double * 2),
                ("kernel_wg_start_us", ctypes.c_double * 2),
                ("kernel_link_gap_us", ctypes.c_double * 2),
                ("kernel_pace_gbps", ctypes.c_double * 2),
                ("kernel_pace_burst_blocks", ctypes.c_double * 2),
                ("kernel_wg_jump_ns", ctypes.c_double * 2),
                ("kernel_cu_exclusive", ctypes.c_double * 2),
                ("kernel_lane_depth", ctypes.c_double * 2)]


class kv_stats_t(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int64 * 2), ("bytes", ctypes.c_int64 * 2),
                ("kernel_launches", ctypes.c_int64 * 2), ("dma_copies", ctypes.c_int64 * 2),
                ("submit_us", ctypes.c_double * 2), ("blocked_us", ctypes.c_double * 2),
                ("last_workgroups", ctypes.c_int64 * 2)]


# Every symbol include/*.h declare, with its ctypes signature.
_P64 = ctypes.POINTER(ctypes.c_int64)
_VP = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
_GEOM = ctypes.POINTER(kv_geometry_t)
_PU64 = ctypes.POINTER(ctypes.c_uint64)
SIGNATURES = {
    "kv_geometry_check": (_I32, [_GEOM]),
    "kv_host_row": (_I64, [_GEOM, _I32, _I32, _I64]),
    "kv_validate": (_I32, [_GEOM, _I32, _P64, _P64, _I64, _I32, _I32, _I32]),
    "kv_count_segments": (_I32, [_GEOM, _P64, _P64, _I64, _I32, _I32, _P64]),
    "kv_count_dma_copies": (_I32, [_GEOM, _P64, _P64, _I64, _I32, _I32, _P64]),
    "kv_pool_create": (_I32, [ctypes.POINTER(kv_pool_desc_t), ctypes.POINTER(_VP)]),
    "kv_pool_create_shared": (_I32, [ctypes.POINTER(kv_pool_desc_t), _VP, ctypes.POINTER(_VP)]),
    "kv_pool_destroy": (_I32, [_VP]),
    "kv_pool_host_ptr": (_VP, [_VP]),
    "kv_pool_host_bytes": (_I64, [_VP]),
    "kv_backup": (_I32, [_VP, _P64, _P64, _I64, _I32, _I32, _VP]),
    "kv_load": (_I32, [_VP, _P64, _P64, _I64, _I32, _I32, _VP]),
    "kv_load_layer": (_I32, [_VP, _I32, _VP]),
    "kv_stage": (_I32, [_VP, _I32, _P64, _I64, _I32, _I32, _VP, _VP]),
    "kv_transfer_noalloc": (_I32, [_VP, _I32, _P64, _P64, _I64, _I32, _I32, _VP]),
    "kv_stream_create": (_I32, [_I32, ctypes.POINTER(_VP)]),
    "kv_stream_destroy": (_I32, [_VP]),
    "kv_set_path": (_I32, [_VP, _I32]),
    "kv_set_direction_path": (_I32, [_VP, _I32, _I32]),
    "kv_last_path": (_I32, [_VP, _I32]),
    "kv_set_calibration": (_I32, [_VP, ctypes.POINTER(kv_calib_t)]),
    "kv_get_calibration": (_I32, [_VP, ctypes.POINTER(kv_calib_t)]),
    "kv_get_stats": (_I32, [_VP, ctypes.POINTER(kv_stats_t)]),
    "kv_default_calibration": (_I32, [ctypes.POINTER(kv_calib_t)]),
    "kv_calibrate_write_pace": (_I32, [_VP, ctypes.c_double, _VP,
                                       ctypes.POINTER(ctypes.c_double)]),
    "kv_model_path": (_I32, [ctypes.POINTER(kv_geometry_t), ctypes.POINTER(kv_calib_t), _I32,
                             _P64, _P64, _I64, _I32, _I32, ctypes.c_uint32,
                             ctypes.POINTER(ctypes.c_double)]),
    "kv_last_error": (ctypes.c_char_p, []),
    "kv_page_hashes": (_I64, [ctypes.POINTER(ctypes.c_int32), _I64, _I32, _PU64]),
    "kv_ghost_create": (_I32, [_I64, ctypes.POINTER(_VP)]),
    "kv_ghost_destroy": (_I32, [_VP]),
    "kv_ghost_insert": (_I32, [_VP, _PU64, _I64]),
    "kv_ghost_reuse_prefix": (_I64, [_VP, _PU64, _I64]),
    "kv_ghost_contains": (_I32, [_VP, ctypes.c_uint64]),
    "kv_ghost_size": (_I64, [_VP]),
    "kv_ghost_snapshot": (_I64, [_VP, _PU64, _I64]),
    "kv_slots_create": (_I32, [_I64, _I32, ctypes.POINTER(_VP)]),
    "kv_slots_destroy": (_I32, [_VP]),
    "kv_slots_alloc": (_I32, [_VP, _I64, _P64]),
    "kv_slots_free": (_I32, [_VP, _P64, _I64]),
    "kv_slots_available": (_I64, [_VP]),
    "kv_slots_snapshot": (_I64, [_VP, _P64, _I64]),
}


def _load():
    # One HIP runtime per process: torch ships its own libamdhip64 (same SONAME,
    # different file name). Loading torch first makes libkvtier.so bind to that
    # already-loaded runtime, so both share one device context; loading the
    # system copy first would leave two runtimes fighting over the GPU.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libkvtier.so is not built (%s). Build it with __graft_entry__.build() or "
            "`python hierarchical_kv_cache_backup_amd/_build.py`; there is no fallback path."
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    return _lib


class KvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERROR_NAMES.get(code, "?"), code, msg))
        self.code = code


def _check(rc):
    if rc < 0:
        raise KvError(rc, kv_last_error())
    return rc


def _idx(a):
    """int64 contiguous numpy copy of an index sequence and its pointer (kept alive by caller)."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a, a.ctypes.data_as(_P64)


def _stream_handle(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def geometry(L, C, R, S_dev, S_host, ps, layout):
    return kv_geometry_t(L, C, R, S_dev, S_host, ps, layout)


# ---- same-name wrappers: return the C status, no exceptions ----------------

def kv_last_error():
    return (_lib.kv_last_error() or b"").decode()


def kv_geometry_check(geom):
    return _lib.kv_geometry_check(ctypes.byref(geom))


def kv_host_row(geom, layer, comp, host_slot):
    return _lib.kv_host_row(ctypes.byref(geom), layer, comp, host_slot)


def kv_validate(geom, direction, dev_idx, host_idx, layer_begin, layer_end, check_unique=True,
                n=None):
    d, dp, h, hp, n = _pair(dev_idx, host_idx, n)
    return _lib.kv_validate(ctypes.byref(geom), direction, dp, hp, n, layer_begin, layer_end,
                            int(check_unique))


def kv_count_segments(geom, dev_idx, host_idx, layer_begin, layer_end):
    """Returns (status, count)."""
    d, dp, h, hp, _ = _pair(dev_idx, host_idx, None)
    out = ctypes.c_int64(-1)
    rc = _lib.kv_count_segments(ctypes.byref(geom), dp, hp, len(d), layer_begin, layer_end,
                                ctypes.byref(out))
    return rc, out.value


def kv_count_dma_copies(geom, dev_idx, host_idx, layer_begin, layer_end):
    d, dp, h, hp, _ = _pair(dev_idx, host_idx, None)
    out = ctypes.c_int64(-1)
    rc = _lib.kv_count_dma_copies(ctypes.byref(geom), dp, hp, len(d), layer_begin, layer_end,
                                  ctypes.byref(out))
    return rc, out.value


def kv_default_calibration():
    """Returns (status, kv_calib_t)."""
    c = kv_calib_t()
    return _lib.kv_default_calibration(ctypes.byref(c)), c


def kv_model_path(geom, calib, direction, dev_idx, host_idx, layer_begin, layer_end, flags=0):
    """Returns (path or status, [kernel_us, dma_us, staged_us])."""
    d, dp, h, hp, _ = _pair(dev_idx, host_idx, None)
    t = (ctypes.c_double * 3)()
    rc = _lib.kv_model_path(ctypes.byref(geom), ctypes.byref(calib), direction, dp, hp, len(d),
                            layer_begin, layer_end, flags, t)
    return rc, list(t)


def kv_pool_create(geom, device_buffer_ptrs, device=0, numa_node=-1, flags=F_CHECK_UNIQUE):
    """Returns (status, handle)."""
    arr = (ctypes.c_void_p * len(device_buffer_ptrs))(*device_buffer_ptrs)
    desc = kv_pool_desc_t(geom, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), device,
                          numa_node, flags)
    h = ctypes.c_void_p()
    rc = _lib.kv_pool_create(ctypes.byref(desc), ctypes.byref(h))
    return rc, h.value


def kv_pool_create_shared(geom, device_buffer_ptrs, group, device=0, flags=F_CHECK_UNIQUE):
    """Returns (status, handle) of a pool sharing `group`'s host pool."""
    arr = (ctypes.c_void_p * len(device_buffer_ptrs))(*device_buffer_ptrs)
    desc = kv_pool_desc_t(geom, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), device,
                          -1, flags)
    h = ctypes.c_void_p()
    rc = _lib.kv_pool_create_shared(ctypes.byref(desc), group, ctypes.byref(h))
    return rc, h.value


def kv_pool_destroy(pool):
    return _lib.kv_pool_destroy(pool)


def kv_pool_host_ptr(pool):
    return _lib.kv_pool_host_ptr(pool)


def kv_pool_host_bytes(pool):
    return _lib.kv_pool_host_bytes(pool)


def _pair(dev_idx, host_idx, n):
    """Both index arrays as int64 with their pointers, and the count the C call
    gets: the arrays must be equally long and n (default: their length) at most
    that long, so the library never reads past either numpy buffer. A negative
    n goes through: the library rejects it (KV_EINVAL) before reading."""
    d, dp = _idx(dev_idx)
    h, hp = _idx(host_idx)
    if len(d) != len(h):
        raise ValueError("dev_idx has %d entries, host_idx %d" % (len(d), len(h)))
    n = len(d) if n is None else int(n)
    if n > len(d):
        raise ValueError("n = %d exceeds the %d index pairs given" % (n, len(d)))
    return d, dp, h, hp, n


def kv_backup(pool, dev_idx, host_idx, layer_begin, layer_end, stream=None, n=None):
    d, dp, h, hp, n = _pair(dev_idx, host_idx, n)
    return _lib.kv_backup(pool, dp, hp, n, layer_begin, layer_end, _stream_handle(stream))


def kv_load(pool, dev_idx, host_idx, layer_begin, layer_end, stream=None, n=None):
    d, dp, h, hp, n = _pair(dev_idx, host_idx, n)
    return _lib.kv_load(pool, dp, hp, n, layer_begin, layer_end, _stream_handle(stream))


def kv_transfer_noalloc(pool, direction, dev_idx, host_idx, layer_begin, layer_end, stream=None,
                        n=None):
    d, dp, h, hp, n = _pair(dev_idx, host_idx, n)
    return _lib.kv_transfer_noalloc(pool, direction, dp, hp, n, layer_begin, layer_end,
                                    _stream_handle(stream))


def kv_stage(pool, direction, dev_idx, layer_begin, layer_end, stage_ptr, stream=None, n=None):
    d, dp = _idx(dev_idx)
    n = len(d) if n is None else int(n)
    if n > len(d):
        raise ValueError("n = %d exceeds the %d device slots given" % (n, len(d)))
    return _lib.kv_stage(pool, direction, dp, n, layer_begin, layer_end, stage_ptr,
                         _stream_handle(stream))


def kv_load_layer(pool, layer, compute_stream=None):
    return _lib.kv_load_layer(pool, layer, _stream_handle(compute_stream))


def kv_stream_create(device=0):
    """Returns (status, hipStream_t handle as int)."""
    h = ctypes.c_void_p()
    rc = _lib.kv_stream_create(device, ctypes.byref(h))
    return rc, h.value


def kv_stream_destroy(stream):
    return _lib.kv_stream_destroy(stream)


class Stream:
    """A stream with a hardware queue of its own (kv_stream_create), usable
    wherever the binding takes a stream; `.torch` is the same stream as a
    torch.cuda.ExternalStream. Destroyed by close()."""

    def __init__(self, device=0):
        import torch
        rc, h = kv_stream_create(device)
        _check(rc)
        self.cuda_stream = h
        self.torch = torch.cuda.ExternalStream(h, device=torch.device("cuda", device))

    def synchronize(self):
        self.torch.synchronize()

    def close(self):
        if self.cuda_stream:
            h, self.cuda_stream = self.cuda_stream, None
            _check(kv_stream_destroy(h))


def kv_set_path(pool, path):
    return _lib.kv_set_path(pool, path)


def kv_set_direction_path(pool, direction, path):
    return _lib.kv_set_direction_path(pool, direction, path)


def kv_last_path(pool, direction):
    return _lib.kv_last_path(pool, direction)


def kv_set_calibration(pool, calib):
    return _lib.kv_set_calibration(pool, ctypes.byref(calib))


def kv_get_calibration(pool):
    c = kv_calib_t()
    rc = _lib.kv_get_calibration(pool, ctypes.byref(c))
    return rc, c


def kv_calibrate_write_pace(pool, fraction=0.98, stream=None):
    """Returns (status, measured D2H GB/s)."""
    g = ctypes.c_double(0.0)
    rc = _lib.kv_calibrate_write_pace(pool, float(fraction), _stream_handle(stream),
                                      ctypes.byref(g))
    return rc, g.value


def kv_get_stats(pool):
    s = kv_stats_t()
    rc = _lib.kv_get_stats(pool, ctypes.byref(s))
    return rc, s


# ---- convenience object over torch device buffers ------------------------------

def _u64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint64))
    return a, a.ctypes.data_as(_PU64)


def kv_page_hashes(tokens, page_size):
    """Page-boundary hashes of a token sequence (uint64 numpy array)."""
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    out = np.zeros(max(t.size // max(int(page_size), 1), 1), dtype=np.uint64)
    rc = _lib.kv_page_hashes(t.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), t.size,
                             int(page_size), out.ctypes.data_as(_PU64))
    _check(rc)
    return out[:rc]


def kv_ghost_create(capacity):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    rc = _lib.kv_ghost_create(int(capacity), ctypes.byref(h))
    return rc, h.value


def kv_ghost_destroy(g):
    return _lib.kv_ghost_destroy(g)


def kv_ghost_insert(g, hashes):
    a, p = _u64(hashes)
    return _lib.kv_ghost_insert(g, p, a.size)


def kv_ghost_reuse_prefix(g, hashes):
    a, p = _u64(hashes)
    return _lib.kv_ghost_reuse_prefix(g, p, a.size)


def kv_ghost_contains(g, h):
    return _lib.kv_ghost_contains(g, int(h) & 0xFFFFFFFFFFFFFFFF)


def kv_ghost_size(g):
    return _lib.kv_ghost_size(g)


def kv_ghost_snapshot(g, max_entries):
    out = np.zeros(max(int(max_entries), 1), dtype=np.uint64)
    rc = _lib.kv_ghost_snapshot(g, out.ctypes.data_as(_PU64), int(max_entries))
    _check(rc)
    return out[:rc]


class GhostList:
    """The Ghost List of evicted page hashes (kv_ghost_*)."""

    def __init__(self, capacity):
        rc, h = kv_ghost_create(capacity)
        _check(rc)
        self.handle = h
        self.capacity = int(capacity)

    def insert(self, hashes):
        _check(kv_ghost_insert(self.handle, hashes))

    def reuse_prefix(self, hashes):
        return _check(kv_ghost_reuse_prefix(self.handle, hashes))

    def contains(self, h):
        return bool(_check(kv_ghost_contains(self.handle, h)))

    def size(self):
        return _check(kv_ghost_size(self.handle))

    def order(self):
        return [int(x) for x in kv_ghost_snapshot(self.handle, self.capacity)]

    def close(self):
        if self.handle:
            h, self.handle = self.handle, None
            kv_ghost_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_slots_create(num_pages, policy):
    """Returns (status, handle)."""
    h = ctypes.c_void_p()
    rc = _lib.kv_slots_create(int(num_pages), int(policy), ctypes.byref(h))
    return rc, h.value


def kv_slots_destroy(a):
    return _lib.kv_slots_destroy(a)


def kv_slots_alloc(a, n):
    """Returns (status, int64 numpy array of the pages taken)."""
    out = np.zeros(max(int(n), 1), dtype=np.int64)
    rc = _lib.kv_slots_alloc(a, int(n), out.ctypes.data_as(_P64))
    return rc, (out[:int(n)] if rc == OK else out[:0])


def kv_slots_free(a, pages):
    p, pp = _idx(pages)
    return _lib.kv_slots_free(a, pp, p.size)


def kv_slots_available(a):
    return _lib.kv_slots_available(a)


def kv_slots_snapshot(a, max_entries):
    out = np.zeros(max(int(max_entries), 1), dtype=np.int64)
    rc = _lib.kv_slots_snapshot(a, out.ctypes.data_as(_P64), int(max_entries))
    _check(rc)
    return out[:rc]


class HostPages:
    """Page allocator of the host pool with a FIFO or LIFO free list (kv_slots_*)."""

    def __init__(self, num_pages, policy=FREE_FIFO):
        rc, h = kv_slots_create(num_pages, policy)
        _check(rc)
        self.handle = h
        self.num_pages = int(num_pages)

    def alloc(self, n):
        rc, pages = kv_slots_alloc(self.handle, n)
        _check(rc)
        return pages

    def free(self, pages):
        _check(kv_slots_free(self.handle, pages))

    def available(self):
        return _check(kv_slots_available(self.handle))

    def order(self):
        return kv_slots_snapshot(self.handle, self.num_pages)

    def close(self):
        if self.handle:
            h, self.handle = self.handle, None
            kv_slots_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KvPool:
    """Owns a library pool over L*C torch uint8 device tensors (borrowed: kept
    referenced here so they outlive the pool). Methods raise KvError on failure."""

    def __init__(self, geom, device_tensors, device=0, numa_node=-1, flags=F_CHECK_UNIQUE,
                 share_with=None):
        """share_with: another KvPool whose host pool this one shares
        (kv_pool_create_shared); numa_node is then ignored."""
        self.geom = geom
        self.tensors = list(device_tensors)
        assert len(self.tensors) == geom.num_layers * geom.num_components
        ptrs = [t.data_ptr() for t in self.tensors]
        if share_with is None:
            rc, h = kv_pool_create(geom, ptrs, device, numa_node, flags)
        else:
            rc, h = kv_pool_create_shared(geom, ptrs, share_with.handle, device, flags)
        _check(rc)
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            rc = kv_pool_destroy(h)
            self.tensors = []
            _check(rc)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def host_array(self):
        """numpy uint8 view of the host pool (CPU address; valid until close)."""
        n = kv_pool_host_bytes(self.handle)
        buf = (ctypes.c_uint8 * n).from_address(kv_pool_host_ptr(self.handle))
        return np.frombuffer(buf, dtype=np.uint8)

    def backup(self, dev_idx, host_idx, layer_begin=0, layer_end=None, stream=None):
        le = self.geom.num_layers if layer_end is None else layer_end
        _check(kv_backup(self.handle, dev_idx, host_idx, layer_begin, le, stream))

    def load(self, dev_idx, host_idx, layer_begin=0, layer_end=None, stream=None):
        le = self.geom.num_layers if layer_end is None else layer_end
        _check(kv_load(self.handle, dev_idx, host_idx, layer_begin, le, stream))

    def stage(self, direction, dev_idx, stage, layer_begin=0, layer_end=None, stream=None):
        """Packs (direction 0) or unpacks (1) the rows of dev_idx between the
        device buffers and `stage` (a torch uint8 device tensor) in host order."""
        le = self.geom.num_layers if layer_end is None else layer_end
        _check(kv_stage(self.handle, direction, dev_idx, layer_begin, le, stage.data_ptr(),
                        stream))

    def load_layer(self, layer, compute_stream=None):
        _check(kv_load_layer(self.handle, layer, compute_stream))

    def set_path(self, path, direction=None):
        """Forces a path for both directions, or for `direction` only."""
        if direction is None:
            _check(kv_set_path(self.handle, path))
        else:
            _check(kv_set_direction_path(self.handle, direction, path))

    def last_path(self, direction):
        return kv_last_path(self.handle, direction)

    def calibration(self):
        rc, c = kv_get_calibration(self.handle)
        _check(rc)
        return c

    def set_calibration(self, c):
        _check(kv_set_calibration(self.handle, c))

    def calibrate_write_pace(self, fraction=0.98, stream=None):
        """Measures the D2H link into this pool's host pool (overwriting its
        start) and paces kernel write-backs at `fraction` of it; returns GB/s."""
        rc, gbps = kv_calibrate_write_pace(self.handle, fraction, stream)
        _check(rc)
        return gbps

    def stats(self):
        rc, s = kv_get_stats(self.handle)
        _check(rc)
        return s
