"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong index or stride, a
transposed operand, an off-by-one bound) in a temporary copy of
oracle/kv_oracle.c, builds it with gcc and runs the pin battery against it: at
least one pin has to fail. The committed oracle itself must pass the whole
battery. Mistakes are planted only in copies, on the CPU.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

_HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (_HERE, os.path.dirname(_HERE)):  # the child process runs this file directly
    if _p not in sys.path:
        sys.path.insert(0, _p)

import oracle  # noqa: E402
from oracle import np_ref, Geometry, LAYOUTS, LAYER_FIRST, PAGE_FIRST, PAGE_FIRST_DIRECT  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "kv_oracle.c")

from test_oracle import parse_layout_golden, bufs_of, stack_bufs  # noqa: E402

MUTANTS = [
    ("layer_first comp stride", "int64_t comp_block = (int64_t)c * S_host;",
     "int64_t comp_block = (int64_t)c * L;"),
    ("page_first dropped factor", "int64_t token_block = h * L * C;",
     "int64_t token_block = h * L;"),
    ("page_first layer stride", "int64_t layer_block = (int64_t)l * C;",
     "int64_t layer_block = (int64_t)l;"),
    ("direct page stride", "int64_t page_block = page * L * C * ps;",
     "int64_t page_block = page * L * ps;"),
    ("direct layer stride", "int64_t layer_block = (int64_t)l * C * ps;",
     "int64_t layer_block = (int64_t)l * ps;"),
    ("direct offset/page swap", "int64_t offset = h % ps;", "int64_t offset = h / ps;"),
    ("direct comp term dropped", "return page_block + layer_block + comp_block + offset;",
     "return page_block + layer_block + offset;"),
    ("backup reads host index", "const uint8_t *src = dev_bufs[l * C + c] + dev_idx[i] * R;",
     "const uint8_t *src = dev_bufs[l * C + c] + host_idx[i] * R;"),
    ("load buffer index transposed", "uint8_t *dst = dev_bufs[l * C + c] + dev_idx[i] * R;",
     "uint8_t *dst = dev_bufs[c * L + l] + dev_idx[i] * R;"),
    ("segments ignore device", "int dev_continues = (dev_idx[i] == dev_idx[i - 1] + 1);",
     "int dev_continues = 1;"),
    ("segments host off by one", "int host_continues = (this_host == prev_host + 1);",
     "int host_continues = (this_host == prev_host);"),
    ("layer range upper bound", "if (l0 < 0 || l0 > l1 || l1 > L) return KVO_EINVAL;",
     "if (l0 < 0 || l0 > l1 || l1 >= L) return KVO_EINVAL;"),
    ("device range off by one", "if (dev_idx[i] < 0 || dev_idx[i] >= S_dev) return KVO_ERANGE;",
     "if (dev_idx[i] < 0 || dev_idx[i] > S_dev) return KVO_ERANGE;"),
    ("duplicate check on source", "const int64_t *dst = (direction == 0) ? host_idx : dev_idx;",
     "const int64_t *dst = (direction == 0) ? dev_idx : host_idx;"),
    ("page divisibility unchecked", "if (S_host % ps != 0) return KVO_EINVAL;", ""),
]


def battery(o):
    """Runs every pin against oracle build `o`; returns the names of failed pins."""
    failed = []

    def pin(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # a crash or assertion counts as a caught mistake
            failed.append(name)

    def golden_orders():
        for (L, C, S_host, ps), rows in parse_layout_golden().items():
            for layout, row, l, c, h in rows:
                if o.host_row(Geometry(L, C, 16, S_host, S_host, ps, layout), l, c, h) != row:
                    return False
        return True

    def pages_example():
        with open(os.path.join(HERE, "golden", "segment_counts.json")) as f:
            gd = json.load(f)
        n = gd["tokens"]
        d = np.arange(n) + 100
        h = np.arange(n)
        g = Geometry(gd["layers"], 1, gd["row_bytes"], n + 100, n, gd["page_size"],
                     PAGE_FIRST_DIRECT)
        lf = g.replace(layout=LAYER_FIRST)
        return (o.count_segments(g, d, h) == gd["page_first_direct_segments"]
                and o.count_segments(lf, d, h) == gd["layer_first_segments"])

    def numpy_equivalence():
        for seed in range(6):
            rng = np.random.default_rng(seed)
            for layout in LAYOUTS:
                g = Geometry(3, 2, 32, 40, 24, 4, layout)
                dev = rng.integers(0, 256, size=(3, 2, 40, 32), dtype=np.uint8)
                n = 13
                d = rng.choice(40, n, replace=False)
                h = rng.choice(24, n, replace=False)
                host = np.full(g.host_bytes(), 0xA5, np.uint8)
                ref = host.copy()
                if o.backup(g, bufs_of(dev), host, d, h, 0, 3) != 0:
                    return False
                np_ref.backup(dev, ref, layout, 3, 2, 24, 4, 32, d, h, 0, 3)
                if not np.array_equal(host, ref):
                    return False
                src = rng.integers(0, 256, size=g.host_bytes(), dtype=np.uint8)
                bufs = bufs_of(dev)
                if o.load(g, bufs, src, d, h, 1, 3) != 0:
                    return False
                want = dev.copy()
                np_ref.load(want, src, layout, 3, 2, 24, 4, 32, d, h, 1, 3)
                if not np.array_equal(stack_bufs(bufs, g), want):
                    return False
                if o.count_segments(g, d, h) != np_ref.count_segments(layout, 3, 2, 24, 4, d, h):
                    return False
                sd, sh = np.sort(d), np.sort(h)
                if o.count_segments(g, sd, sh) != np_ref.count_segments(layout, 3, 2, 24, 4,
                                                                        sd, sh):
                    return False
        return True

    def validation():
        g = Geometry(4, 2, 32, 10, 8, 4, PAGE_FIRST)
        checks = [
            o.validate(g, 0, [1, 2, 3], [0, 5, 7], 0, 4) == 0,
            o.validate(g, 0, [1, 2, 3], [0, 5, 7], 0, 5) == -1,
            o.validate(g, 0, [10, 1, 2], [0, 5, 7], 0, 4) == -2,
            o.validate(g, 1, [1, 1, 2], [0, 5, 7], 0, 4) == -3,
            o.validate(g, 0, [1, 2, 3], [3, 4, 3], 0, 4) == -3,
            o.validate(g, 0, [1, 1, 2], [0, 5, 7], 0, 4) == 0,
            o.check_geometry(g.replace(S_host=10)) == -1,
        ]
        return all(checks)

    pin("golden storage orders", golden_orders)
    pin("pages' segment example", pages_example)
    pin("numpy derivation", numpy_equivalence)
    pin("validation codes", validation)
    return failed


def _battery_in_child(lib):
    return subprocess.run([sys.executable, os.path.abspath(__file__), lib], capture_output=True,
                          text=True, timeout=300, cwd=os.path.dirname(HERE))


def test_committed_oracle_passes_every_pin():
    assert battery(oracle.default()) == []
    # the child-process harness itself must pass on the committed oracle,
    # else a broken harness would make every planted mistake look caught
    res = _battery_in_child(oracle.default().path)
    assert res.returncode == 0, res.stdout + res.stderr


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    """The battery runs in a child process: a planted stride mistake can write
    outside the arrays, and a crash there counts as a caught mistake without
    corrupting this process."""
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"), werror=False)
    res = _battery_in_child(lib)
    assert "No module named" not in res.stderr, res.stderr
    assert res.returncode != 0, "planted mistake '%s' passed every pin" % name


if __name__ == "__main__":
    # child process: run the battery against the oracle build given on the
    # command line; exit 0 only if every pin passed
    failed = battery(oracle.Oracle(sys.argv[1]))
    print("failed pins:", failed)
    sys.exit(1 if failed else 0)
