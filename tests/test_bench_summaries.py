"""The interference study's summary (bench.py --summarize-interference), on
rocprofv3-shaped CSV files written here: the reduction kernel's dispatches are
cut into the phases the consumer recorded, in dispatch order, and each phase
reports per-dispatch medians and ratios. No GPU."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

REDUCE = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<long>>(...)"
ADD = "void at::native::vectorized_elementwise_kernel<4, at::native::AddFunctor<long>>(...)"


def write_run(d, phases, value_of, dur_of, drop_last=False):
    """A consumer directory: consumer.json plus counter and kernel-trace CSVs in
    which every reduction is followed by an add, both with counters."""
    os.makedirs(os.path.join(d, "prof"))
    with open(os.path.join(d, "consumer.json"), "w") as f:
        json.dump({"phases": [{"phase": p, "reduce_dispatches": k} for p, k in phases],
                   "loader": {"x": {"h2d_gbps": 1.0}}}, f)
    counters, trace = [], []
    did = 0
    for p, k in phases:
        for i in range(k):
            for name in (REDUCE, ADD):
                did += 1
                if drop_last and p == phases[-1][0] and i == k - 1 and name == REDUCE:
                    continue
                for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_LEVEL_sum"):
                    counters.append({"Correlation_Id": did, "Dispatch_Id": did,
                                     "Kernel_Name": name, "Counter_Name": c,
                                     "Counter_Value": value_of(p, i, c)})
                trace.append({"Dispatch_Id": did, "Kernel_Name": name,
                              "Start_Timestamp": 10 ** 6 * did,
                              "End_Timestamp": 10 ** 6 * did + dur_of(p, i)})
    for fname, rows in (("kv_counter_collection.csv", counters), ("kv_kernel_trace.csv", trace)):
        with open(os.path.join(d, "prof", fname), "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=list(rows[0]))
            w.writeheader()
            w.writerows(rows)


def table(text):
    lines = [l for l in text.splitlines() if l.startswith("|")]
    head = [c.strip() for c in lines[0].strip("|").split("|")]
    return {cells[0]: dict(zip(head, cells))
            for cells in ([c.strip() for c in l.strip("|").split("|")] for l in lines[2:])}


def test_phases_split_in_dispatch_order(tmp_path, capsys):
    phases = [("warmup", 2), ("alone", 5), ("beside", 5)]
    # requests 100 per dispatch; in-flight level 100 * latency, latency 10 alone
    # and 30 beside; durations 50 us alone, 100 us beside
    lat = {"warmup": 10.0, "alone": 10.0, "beside": 30.0}

    def value(p, i, c):
        return 100.0 if c == "TCC_EA0_RDREQ_sum" else 100.0 * lat[p] + i

    def dur(p, i):
        return 100000 if p == "beside" else 50000

    d = str(tmp_path / "run")
    write_run(d, phases, value, dur)
    bench.summarize_interference([d])
    t = table(capsys.readouterr().out)
    assert list(t) == ["warmup", "alone", "beside"]
    assert float(t["alone"]["duration_us"]) == 50.0
    assert float(t["beside"]["duration_us"]) == 100.0
    # per-dispatch ratio, then the median over the phase's 5 dispatches (i = 2)
    assert float(t["alone"]["ea_read_latency_cycles"]) == pytest.approx(10.02)
    assert float(t["beside"]["ea_read_latency_cycles"]) == pytest.approx(30.02)


def test_count_mismatch_is_refused(tmp_path):
    d = str(tmp_path / "run")
    write_run(d, [("alone", 3), ("beside", 3)], lambda p, i, c: 1.0, lambda p, i: 1000,
              drop_last=True)
    with pytest.raises(SystemExit):
        bench.summarize_interference([d])
