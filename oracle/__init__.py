"""CPU oracle for the cross-tier KV transfer — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The library and its Python binding never
do, and nothing here imports them: the two share no code.

Two independent derivations of the same bytes:

* ``kv_oracle.c`` (loaded through ctypes): validation, the host-row address map
  written out per layout, backup/load as nested loops of ``memcpy`` per row, and
  the per-(layer, component) DMA segment count. Pages: "Tuning SGLang HiCache L2
  on Kunlunxin P800/P900" section 2.1 (layouts, segment counting) and "HiCache
  system design" section "data transfer optimisation" (page_first granularity).
* ``np_ref`` (NumPy): the same copies obtained by viewing the host pool in each
  layout's dimension order with ``reshape``/``transpose`` and assigning through
  fancy indexing; it never evaluates a host-row formula.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import np_ref  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv_oracle.c")
_LIB = os.path.join(_HERE, "libkv_oracle.so")

OK, EINVAL, ERANGE, EDUP = 0, -1, -2, -3
LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT = 0, 1, 2
LAYOUTS = (LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT)


def build(src=_SRC, out=_LIB, werror=True):
    """Compile kv_oracle.c (or a given copy of it) with gcc into a shared library."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra"] + (["-Werror"] if werror else []) + [
        "-shared", "-fPIC", "-o", out + ".tmp", src]
    subprocess.check_call(cmd)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes binding of one build of kv_oracle.c (the default build, or a test's
    deliberately mutated copy)."""

    def __init__(self, path):
        L = ctypes.CDLL(path)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        p64 = ctypes.POINTER(ctypes.c_int64)
        pp8 = ctypes.POINTER(ctypes.c_void_p)
        geom = [i32, i32, i64, i64, i64, i32, i32]
        L.kvo_check_geometry.argtypes = geom
        L.kvo_check_geometry.restype = i32
        L.kvo_host_row.argtypes = [i32, i32, i32, i64, i32, i32, i32, i64]
        L.kvo_host_row.restype = i64
        L.kvo_validate.argtypes = geom + [i32, p64, p64, i64, i32, i32, i32]
        L.kvo_validate.restype = i32
        L.kvo_backup.argtypes = geom + [pp8, ctypes.c_void_p, p64, p64, i64, i32, i32, i32]
        L.kvo_backup.restype = i32
        L.kvo_load.argtypes = geom + [pp8, ctypes.c_void_p, p64, p64, i64, i32, i32, i32]
        L.kvo_load.restype = i32
        L.kvo_count_segments.argtypes = geom + [p64, p64, i64, i32, i32]
        L.kvo_count_segments.restype = i64
        self.c = L
        self.path = path

    def check_geometry(self, g):
        return self.c.kvo_check_geometry(*g.args())

    def host_row(self, g, l, c, h):
        return self.c.kvo_host_row(g.layout, g.L, g.C, g.S_host, g.ps, l, c, h)

    def validate(self, g, direction, dev_idx, host_idx, l0, l1, check_unique=True):
        d, dp = _idx(dev_idx)
        h, hp = _idx(host_idx)
        return self.c.kvo_validate(*g.args(), direction, dp, hp, len(d), l0, l1,
                                   int(check_unique))

    def backup(self, g, dev_bufs, host, dev_idx, host_idx, l0=0, l1=None, check_unique=True):
        """D2H on host mirrors: dev_bufs = L*C uint8 arrays, host = uint8 array (modified)."""
        l1 = g.L if l1 is None else l1
        d, dp = _idx(dev_idx)
        h, hp = _idx(host_idx)
        assert host.dtype == np.uint8 and host.flags.c_contiguous and host.size == g.host_bytes()
        bufs = _bufs(dev_bufs)
        return self.c.kvo_backup(*g.args(), bufs, host.ctypes.data, dp, hp, len(d), l0, l1,
                                 int(check_unique))

    def load(self, g, dev_bufs, host, dev_idx, host_idx, l0=0, l1=None, check_unique=True):
        """H2D on host mirrors: dev_bufs (modified) <- host."""
        l1 = g.L if l1 is None else l1
        d, dp = _idx(dev_idx)
        h, hp = _idx(host_idx)
        assert host.dtype == np.uint8 and host.flags.c_contiguous and host.size == g.host_bytes()
        bufs = _bufs(dev_bufs)
        return self.c.kvo_load(*g.args(), bufs, host.ctypes.data, dp, hp, len(d), l0, l1,
                               int(check_unique))

    def count_segments(self, g, dev_idx, host_idx, l0=0, l1=None):
        l1 = g.L if l1 is None else l1
        d, dp = _idx(dev_idx)
        h, hp = _idx(host_idx)
        return self.c.kvo_count_segments(*g.args(), dp, hp, len(d), l0, l1)


_default = None


def default():
    """The oracle built from kv_oracle.c; compiled first only if never built."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


class Geometry:
    """Pool geometry: L layers, C components, R row bytes, S_dev/S_host slots, ps, layout."""

    def __init__(self, L, C, R, S_dev, S_host, ps, layout):
        self.L, self.C, self.R = int(L), int(C), int(R)
        self.S_dev, self.S_host, self.ps, self.layout = int(S_dev), int(S_host), int(ps), int(layout)

    def args(self):
        return (self.L, self.C, self.R, self.S_dev, self.S_host, self.ps, self.layout)

    def host_bytes(self):
        return self.L * self.C * self.S_host * self.R

    def replace(self, **kw):
        d = dict(L=self.L, C=self.C, R=self.R, S_dev=self.S_dev, S_host=self.S_host,
                 ps=self.ps, layout=self.layout)
        d.update(kw)
        return Geometry(**d)

    def __repr__(self):
        return ("Geometry(L=%d, C=%d, R=%d, S_dev=%d, S_host=%d, ps=%d, layout=%d)"
                % self.args())


def _idx(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _bufs(dev_bufs):
    """dev_bufs: sequence of L*C contiguous uint8 arrays (S_dev*R bytes each)."""
    for b in dev_bufs:
        assert b.dtype == np.uint8 and b.flags.c_contiguous
    arr = (ctypes.c_void_p * len(dev_bufs))(*[b.ctypes.data for b in dev_bufs])
    return arr


def check_geometry(g):
    return default().check_geometry(g)


def host_row(g, l, c, h):
    return default().host_row(g, l, c, h)


def validate(g, direction, dev_idx, host_idx, l0, l1, check_unique=True):
    return default().validate(g, direction, dev_idx, host_idx, l0, l1, check_unique)


def backup(g, dev_bufs, host, dev_idx, host_idx, l0=0, l1=None, check_unique=True):
    return default().backup(g, dev_bufs, host, dev_idx, host_idx, l0, l1, check_unique)


def load(g, dev_bufs, host, dev_idx, host_idx, l0=0, l1=None, check_unique=True):
    return default().load(g, dev_bufs, host, dev_idx, host_idx, l0, l1, check_unique)


def count_segments(g, dev_idx, host_idx, l0=0, l1=None):
    return default().count_segments(g, dev_idx, host_idx, l0, l1)
