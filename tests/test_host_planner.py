"""Host-side checks of libkvtier.so that need no GPU.

* the shared library loads and exports every function include/*.h declares;
* the planner's entry points (address map, validation, segment and copy counts)
  agree with the oracle, element by element;
* a host-compiled replay driver (tests/host/walk_check.cpp, AddressSanitizer +
  UBSan) runs every launch plan of the kernels and of the copy-engine path on
  CPU mirrors and compares the bytes with the oracle;
* the Ghost List and the host page allocator run random operation streams
  under the same sanitizers (tests/host/ghost_check.cpp, slots_check.cpp).
"""
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from oracle import Geometry, LAYOUTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
CSRC = os.path.join(ROOT, "hierarchical_kv_cache_backup_amd", "csrc")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def kvt():
    import hierarchical_kv_cache_backup_amd as kvt
    return kvt


def test_library_exports_every_declared_symbol(kvt):
    names = declared_functions()
    assert len(names) >= 18
    lib = kvt.library()
    for name in names:
        assert hasattr(lib, name), name
        assert name in kvt.SIGNATURES, name
    assert sorted(kvt.SIGNATURES) == names
    out = subprocess.check_output(["nm", "-D", "--defined-only", kvt.LIB_PATH], text=True)
    exported = set(re.findall(r" T (kv_\w+)", out))
    assert set(names) <= exported


def _geom(kvt, g):
    return kvt.geometry(g.L, g.C, g.R, g.S_dev, g.S_host, g.ps, g.layout)


def test_host_row_matches_oracle(kvt):
    rng = np.random.default_rng(0)
    for _ in range(60):
        L, C = int(rng.integers(1, 80)), int(rng.integers(1, 3))
        ps = int(rng.choice([1, 2, 16, 64]))
        g = Geometry(L, C, 16 * int(rng.integers(1, 200)), 1000, ps * int(rng.integers(1, 600)),
                     ps, int(rng.integers(0, 3)))
        kg = _geom(kvt, g)
        for _ in range(40):
            l, c, h = int(rng.integers(0, L)), int(rng.integers(0, C)), int(rng.integers(0, g.S_host))
            assert kvt.kv_host_row(kg, l, c, h) == oracle.host_row(g, l, c, h)
        assert kvt.kv_host_row(kg, L, 0, 0) == kvt.ERANGE
        assert kvt.kv_host_row(kg, 0, 0, g.S_host) == kvt.ERANGE


def test_geometry_and_validation_codes_match_oracle(kvt):
    base = Geometry(4, 2, 32, 10, 8, 4, 1)
    bad = [base.replace(R=24), base.replace(R=0), base.replace(S_host=10), base.replace(ps=0),
           base.replace(L=0), base.replace(C=0), base.replace(layout=3), base.replace(S_dev=0)]
    for g in [base] + bad:
        assert kvt.kv_geometry_check(_geom(kvt, g)) == oracle.check_geometry(g), g
    cases = [([1, 2, 3], [0, 5, 7], 0, 4), ([], [], 0, 4), ([1, 2, 3], [0, 5, 7], 2, 2),
             ([1, 2, 3], [0, 5, 7], -1, 2), ([1, 2, 3], [0, 5, 7], 3, 2),
             ([1, 2, 3], [0, 5, 7], 0, 5), ([10, 1, 2], [0, 5, 7], 0, 4),
             ([-1, 1, 2], [0, 5, 7], 0, 4), ([1, 2, 3], [0, 8, 1], 0, 4),
             ([1, 1, 2], [0, 5, 7], 0, 4), ([1, 2, 3], [3, 4, 3], 0, 4),
             ([1, 2, 3, 4], [3, 3, 1, 9], 0, 4), ([5, 5, 5], [1, 1, 1], 0, 1)]
    kg = _geom(kvt, base)
    for direction in (0, 1):
        for uniq in (True, False):
            for d, h, l0, l1 in cases:
                want = oracle.validate(base, direction, d, h, l0, l1, uniq)
                got = kvt.kv_validate(kg, direction, d, h, l0, l1, uniq)
                assert got == want, (direction, uniq, d, h, l0, l1)
    assert kvt.kv_validate(kg, 0, [1], [1], 0, 1, True, n=-1) == kvt.EINVAL
    # the library's own ceiling on a row (the kernels count a row's chunks in
    # 32 bits); the pages set none, so the oracle takes both
    assert kvt.kv_geometry_check(_geom(kvt, base.replace(R=1 << 30))) == kvt.OK
    assert kvt.kv_geometry_check(_geom(kvt, base.replace(R=(1 << 30) + 16))) == kvt.EINVAL
    rng = np.random.default_rng(1)
    for _ in range(200):
        g = Geometry(int(rng.integers(1, 4)), int(rng.integers(1, 3)), 16, int(rng.integers(1, 9)),
                     4 * int(rng.integers(1, 3)), 4, int(rng.integers(0, 3)))
        n = int(rng.integers(0, 6))
        d = rng.integers(-1, g.S_dev + 1, n)
        h = rng.integers(-1, g.S_host + 1, n)
        l0 = int(rng.integers(-1, g.L + 1))
        l1 = int(rng.integers(-1, g.L + 2))
        for direction in (0, 1):
            assert (kvt.kv_validate(_geom(kvt, g), direction, d, h, l0, l1, True)
                    == oracle.validate(g, direction, d, h, l0, l1, True))


def test_uniqueness_check_on_huge_pools(kvt):
    """Pools with far more slots than a request's positions (2^40 here): the
    duplicate check must not hold memory per slot, and it agrees with the oracle,
    including the position the message names."""
    g = Geometry(1, 1, 16, 1 << 40, 1 << 40, 1, 0)
    kg = _geom(kvt, g)
    rng = np.random.default_rng(5)
    for trial in range(40):
        n = int(rng.integers(2, 3000))
        d = rng.choice(1 << 40, n, replace=False)
        h = rng.choice(1 << 40, n, replace=False)
        if trial % 2:
            j, k = sorted(rng.choice(n, 2, replace=False))
            d[k] = d[j]
            h[k] = h[j]
        for direction in (0, 1):
            want = oracle.validate(g, direction, d, h, 0, 1, True)
            assert kvt.kv_validate(kg, direction, d, h, 0, 1, True) == want
            if want == kvt.EDUP:
                assert ("position %d)" % k) in kvt.kv_last_error()
    # the stamp array and the sorted copy name the same first repeat
    small = Geometry(1, 1, 16, 64, 64, 1, 0)
    for big in (False, True):
        gg = Geometry(1, 1, 16, 1 << 40, 1 << 40, 1, 0) if big else small
        assert kvt.kv_validate(_geom(kvt, gg), 0, [1, 2, 3, 4, 5], [9, 7, 8, 7, 9], 0, 1,
                               True) == kvt.EDUP
        assert "host slot 7 is a destination twice (position 3)" in kvt.kv_last_error()


def test_segment_counts_match_oracle(kvt):
    rng = np.random.default_rng(2)
    for _ in range(150):
        ps = int(rng.choice([1, 2, 4, 16]))
        g = Geometry(int(rng.integers(1, 6)), int(rng.integers(1, 3)), 32, 300,
                     ps * int(rng.integers(1, 20)), ps, int(rng.integers(0, 3)))
        n = int(rng.integers(0, min(g.S_dev, g.S_host) + 1))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            d = rng.choice(g.S_dev, n, replace=False)
            h = rng.choice(g.S_host, n, replace=False)
        elif kind == 1:
            d0 = int(rng.integers(0, g.S_dev - n + 1))
            d = np.arange(d0, d0 + n)
            h = np.arange(n)
        else:  # whole pages in random order on the device
            d = np.arange(n)
            h = np.arange(n)
            pages = rng.permutation(max(1, -(-n // ps)))
            d = np.concatenate([np.arange(p * ps, p * ps + ps) for p in pages])[:n] if n else d
        l0 = int(rng.integers(0, g.L + 1))
        l1 = int(rng.integers(l0, g.L + 1))
        rc, cnt = kvt.kv_count_segments(_geom(kvt, g), d, h, l0, l1)
        assert rc == 0 and cnt == oracle.count_segments(g, d, h, l0, l1)
        rc2, copies = kvt.kv_count_dma_copies(_geom(kvt, g), d, h, l0, l1)
        assert rc2 == 0 and copies <= cnt


def test_pages_example_through_library(kvt):
    """32K tokens, page 64, 78 layers: 39,936 segments page_first_direct, 78 layer_first;
    the copy-engine plan merges page_first_direct's uniform-stride pages into one
    2-D copy per layer. The pool holds exactly these 512 pages, so the 2-D region
    of layer l (512 pitches of 78 x 64 rows from row l x 64) ends l x 64 rows past
    the pool: every layer but the first sends its last page as a call of its own."""
    n = 32768
    d = np.arange(n) + 8192
    h = np.arange(n)
    for layout, segs, copies in ((2, 39936, 1 + 77 * 2), (0, 78, 78)):
        kg = kvt.geometry(78, 1, 1152, 65536, n, 64, layout)
        assert kvt.kv_count_segments(kg, d, h, 0, 78) == (0, segs)
        assert kvt.kv_count_dma_copies(kg, d, h, 0, 78) == (0, copies)
    kg = kvt.geometry(78, 1, 1152, 65536, 2 * n, 64, 2)   # a pool twice the prefix
    assert kvt.kv_count_dma_copies(kg, d, h, 0, 78) == (0, 78)


def test_replay_driver_under_sanitizers(tmp_path):
    obj = tmp_path / "oracle.o"
    exe = tmp_path / "walk_check"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    subprocess.check_call(["gcc", "-O1", "-g", "-c", os.path.join(ROOT, "oracle", "kv_oracle.c"),
                           "-o", str(obj)] + san)
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-I" + os.path.join(ROOT, "include"),
                           "-I" + CSRC, os.path.join(HERE, "host", "walk_check.cpp"),
                           os.path.join(CSRC, "plan.cpp"), str(obj), "-o", str(exe)] + san)
    res = subprocess.run([str(exe), "160"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout


def test_binding_structs_match_header(kvt, tmp_path):
    """The ctypes structures have the header's size and field offsets (a C
    program built against include/kvtier.h prints them)."""
    import ctypes
    structs = {"kv_geometry_t": kvt.kv_geometry_t, "kv_pool_desc_t": kvt.kv_pool_desc_t,
               "kv_calib_t": kvt.kv_calib_t, "kv_stats_t": kvt.kv_stats_t}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "kvtier.h"',
             "int main(void) {"]
    for name, cls in structs.items():
        lines.append('  printf("%s size %%zu\\n", sizeof(%s));' % (name, name))
        for f, _ in cls._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (name, f, name, f))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src),
                           "-o", str(exe)])
    got = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        a, b, v = line.split()
        got[(a, b)] = int(v)
    for name, cls in structs.items():
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)


def test_ghost_list_under_sanitizers(tmp_path):
    exe = tmp_path / "ghost_check"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-I" + os.path.join(ROOT, "include"),
                           os.path.join(HERE, "host", "ghost_check.cpp"),
                           os.path.join(CSRC, "ghost.cpp"), "-o", str(exe), "-lpthread"] + san)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout


def test_host_page_allocator_under_sanitizers(tmp_path):
    exe = tmp_path / "slots_check"
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-I" + os.path.join(ROOT, "include"),
                           os.path.join(HERE, "host", "slots_check.cpp"),
                           os.path.join(CSRC, "slots.cpp"), "-o", str(exe), "-lpthread"] + san)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout


def test_allocator_and_ghost_list_threads_under_tsan(tmp_path):
    """Four threads on one page allocator and on one Ghost List at once, built
    with ThreadSanitizer: no data race, no page handed to two holders, every
    page free at the end, the Ghost List within capacity."""
    exe = tmp_path / "threads_check"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread",
                           "-I" + os.path.join(ROOT, "include"),
                           os.path.join(HERE, "host", "threads_check.cpp"),
                           os.path.join(CSRC, "slots.cpp"), os.path.join(CSRC, "ghost.cpp"),
                           "-o", str(exe), "-lpthread"])
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
    assert "ThreadSanitizer" not in res.stderr, res.stderr


def test_binding_refuses_index_arrays_it_would_read_past(kvt):
    """The same-name wrappers check that dev_idx and host_idx are equally long
    and that n does not exceed them, before the C call reads the arrays."""
    kg = kvt.geometry(2, 1, 16, 8, 8, 4, 0)
    with pytest.raises(ValueError):
        kvt.kv_validate(kg, 0, [1, 2, 3], [1, 2], 0, 1)
    with pytest.raises(ValueError):
        kvt.kv_validate(kg, 0, [1, 2], [1, 2], 0, 1, n=3)
    with pytest.raises(ValueError):
        kvt.kv_count_segments(kg, [1, 2, 3], [1], 0, 1)
    with pytest.raises(ValueError):
        kvt.kv_backup(None, [1, 2], [1], 0, 1)
    with pytest.raises(ValueError):
        kvt.kv_load(None, [1], [1], 0, 1, n=2)
    assert kvt.kv_validate(kg, 0, [1, 2], [1, 2], 0, 1, n=1) == kvt.OK
    assert kvt.kv_validate(kg, 0, [1], [1], 0, 1, n=-1) == kvt.EINVAL


def test_dma_copy_count_splits_regions_past_the_pool(kvt):
    """A 2-D copy whose pitch x height region would end past the host pool or
    the device buffer sends its last line on its own: runs of 16 slots at pitch
    32 from slot 16 of a 640-slot pool are one 2-D copy of 20 lines per buffer
    whose device region ends 16 rows past the buffer (every buffer splits), and
    the last 4 pages of a 78-layer page_first_direct pool are one 4-line copy
    per layer whose host region ends l*64 rows past the pool on layer l (all
    but layer 0 split)."""
    d = np.concatenate([np.arange(s, s + 16) for s in range(16, 640, 32)])
    kg = kvt.geometry(3, 2, 48, 640, 640, 16, 0)
    assert kvt.kv_count_segments(kg, d, d, 0, 3) == (0, 20 * 6)
    assert kvt.kv_count_dma_copies(kg, d, d, 0, 3) == (0, 2 * 6)
    kg = kvt.geometry(3, 2, 48, 656, 640, 16, 0)     # device buffer holds the region
    assert kvt.kv_count_dma_copies(kg, d, d, 0, 3) == (0, 1 * 5 + 2)
    kg = kvt.geometry(78, 1, 16, 256, 512, 64, 2)
    d, h = np.arange(256), np.arange(256, 512)
    assert kvt.kv_count_segments(kg, d, h, 0, 78) == (0, 4 * 78)
    assert kvt.kv_count_dma_copies(kg, d, h, 0, 78) == (0, 1 + 77 * 2)
    assert kvt.kv_count_dma_copies(kg, d, h, 1, 78) == (0, 77 * 2)
    assert kvt.kv_count_dma_copies(kg, d, h, 0, 1) == (0, 1)
