"""Pins of the free-list oracle (oracle/slots.py) against what the pages fix,
independent of the oracle's own list splicing: hand-worked traces
(tests/golden/free_list_trace.txt), a second model that orders free pages by
the time they were freed, the partition invariant, LIFO's reuse of the batch
freed last, the closed forms of how many distinct pages a steady churn
touches under each policy, and refused calls leaving the state unchanged.
Planted mistakes in copies of the oracle must each fail one of these pins.
Source: "Tuning SGLang HiCache L2 on Kunlunxin P800/P900", section 2.4 ("LIFO
free list"); "Baidu's KVCache Overhaul", "LIFO slot allocation"."""
import os

import numpy as np
import pytest

from oracle import slots

HERE = os.path.dirname(os.path.abspath(__file__))
STATUS = {"ENOMEM": slots.ENOMEM, "ERANGE": slots.ERANGE, "EINVAL": slots.EINVAL}


def parse_traces():
    traces, cur = {}, None
    for line in open(os.path.join(HERE, "golden", "free_list_trace.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.startswith("["):
            name, pages = line.strip("[]").split()
            cur = traces.setdefault(name, {"pages": int(pages), "ops": []})
            continue
        lhs, rhs = line.split("=>")
        result, after = (x.strip() for x in rhs.split(";"))
        op, *args = lhs.split()
        cur["ops"].append((op, [int(a) for a in args], result,
                           [] if after == "-" else [int(x) for x in after.split()]))
    return traces


# ---- pins, each taking the allocator class so planted mistakes can be run --------

def pin_golden(cls):
    for name, tr in parse_traces().items():
        fl = cls(tr["pages"], slots.FIFO if name == "FIFO" else slots.LIFO)
        for op, args, result, after in tr["ops"]:
            if op == "alloc":
                rc, got = fl.alloc(args[0])
                if result in STATUS:
                    assert rc == STATUS[result], (name, op, args)
                else:
                    assert rc == slots.OK and got == ([] if result == "-" else
                                                      [int(x) for x in result.split()]), \
                        (name, op, args, got)
            else:
                rc = fl.release(args)
                assert rc == (slots.OK if result == "ok" else STATUS[result]), (name, op, args)
            assert fl.order() == after, (name, op, args, fl.order())


class StampModel:
    """Second model of the same allocator: every free page carries a stamp (the
    time it became free, its place in its batch); an allocation hands out the
    free pages with the smallest stamps (FIFO) or, batch by batch, the latest
    batch first (LIFO). The initial pages count as one batch freed before time 0."""

    def __init__(self, num_pages, policy):
        self.policy = policy
        self.num_pages = num_pages
        self.stamp = {p: (-1, p) for p in range(num_pages)}
        self.t = 0

    def key(self, p):
        t, i = self.stamp[p]
        return (t, i) if self.policy == slots.FIFO else (-t, i)

    def alloc(self, k):
        if k > len(self.stamp):
            return None
        out = sorted(self.stamp, key=self.key)[:k]
        for p in out:
            del self.stamp[p]
        return out

    def release(self, pages):
        for i, p in enumerate(pages):
            self.stamp[p] = (self.t, i)
        self.t += 1

    def order(self):
        return sorted(self.stamp, key=self.key)


def random_ops(rng, num_pages, steps):
    """Random valid alloc/free operations (frees take random subsets of the
    allocated pages, in random order). Yields ("alloc", k) / ("free", batch)."""
    held = []
    for _ in range(steps):
        if held and rng.random() < 0.5:
            m = int(rng.integers(1, len(held) + 1))
            pick = rng.permutation(len(held))[:m]
            batch = [held[j] for j in pick]
            held = [h for j, h in enumerate(held) if j not in set(pick.tolist())]
            yield "free", batch
        else:
            k = int(rng.integers(0, num_pages + 1))
            got = yield "alloc", k
            if got:
                held.extend(got)


def drive(fl, gen):
    """Runs random_ops against an allocator; returns (op, arg, status, pages allocated,
    free list after, free count after) per operation."""
    out = []
    try:
        op, arg = next(gen)
        while True:
            if op == "alloc":
                rc, got = fl.alloc(arg)
                out.append((op, arg, rc, list(got), fl.order(), fl.available()))
                op, arg = gen.send(got if rc == slots.OK else [])
            else:
                rc = fl.release(arg)
                out.append((op, list(arg), rc, None, fl.order(), fl.available()))
                op, arg = next(gen)
    except StopIteration:
        pass
    return out


def pin_stamp_model(cls):
    for seed in range(60):
        rng = np.random.default_rng(seed)
        P = int(rng.integers(1, 12))
        for policy in (slots.FIFO, slots.LIFO):
            fl = cls(P, policy)
            model = StampModel(P, policy)
            for op, arg, rc, got, order, _ in drive(fl, random_ops(np.random.default_rng(seed), P, 40)):
                if op == "alloc":
                    want = model.alloc(arg)
                    if want is None:
                        assert rc == slots.ENOMEM, (seed, policy, arg)
                    else:
                        assert rc == slots.OK and got == want, (seed, policy, arg, got, want)
                else:
                    assert rc == slots.OK, (seed, policy, arg)
                    model.release(arg)
                assert order == model.order(), (seed, policy)


def pin_partition(cls):
    for seed in range(30):
        rng = np.random.default_rng(100 + seed)
        P = int(rng.integers(1, 20))
        for policy in (slots.FIFO, slots.LIFO):
            fl = cls(P, policy)
            held = set()
            for op, arg, rc, got, order, avail in drive(fl, random_ops(rng, P, 50)):
                if rc == slots.OK:
                    if op == "alloc":
                        assert not held & set(got)
                        held |= set(got)
                    else:
                        held -= set(arg)
                assert len(order) == len(set(order))
                assert set(order) | held == set(range(P)) and not set(order) & held
                assert avail == P - len(held)


def pin_lifo_reuses_last_batch(cls):
    rng = np.random.default_rng(7)
    for _ in range(40):
        P = int(rng.integers(2, 30))
        fl = cls(P, slots.LIFO)
        rc, got = fl.alloc(int(rng.integers(1, P + 1)))
        assert rc == slots.OK
        for _ in range(5):
            batch = [int(x) for x in rng.permutation(got)[:int(rng.integers(1, len(got) + 1))]]
            assert fl.release(batch) == slots.OK
            rc, again = fl.alloc(len(batch))
            assert rc == slots.OK and again == batch


def churn_distinct(cls, policy, P, W, k, T):
    """W live requests of k pages each; every round frees the oldest request and
    allocates a new one. Returns the number of distinct pages ever handed out."""
    fl = cls(P, policy)
    live, touched = [], set()
    for _ in range(W):
        rc, got = fl.alloc(k)
        assert rc == slots.OK
        live.append(got)
        touched |= set(got)
    for _ in range(T):
        assert fl.release(live.pop(0)) == slots.OK
        rc, got = fl.alloc(k)
        assert rc == slots.OK
        live.append(got)
        touched |= set(got)
    return len(touched)


def pin_churn_closed_forms(cls):
    # LIFO keeps reusing the W*k pages of the working set; FIFO hands out fresh
    # pages until it has walked the whole pool: min(P, (W+T)*k)
    for P, W, k, T in ((64, 4, 2, 50), (100, 3, 5, 4), (1000, 10, 16, 30), (48, 6, 8, 0),
                       (256, 1, 64, 10), (30, 2, 3, 100)):
        assert churn_distinct(cls, slots.LIFO, P, W, k, T) == W * k, (P, W, k, T)
        assert churn_distinct(cls, slots.FIFO, P, W, k, T) == min(P, (W + T) * k), (P, W, k, T)


def pin_refusals_change_nothing(cls):
    for policy in (slots.FIFO, slots.LIFO):
        fl = cls(10, policy)
        rc, got = fl.alloc(6)
        assert rc == slots.OK
        assert fl.release([got[0]]) == slots.OK
        before = fl.order()
        assert fl.alloc(len(before) + 1) == (slots.ENOMEM, [])
        assert fl.release([got[1], got[0]]) == slots.EINVAL      # got[0] is free
        assert fl.release([got[1], got[2], got[1]]) == slots.EINVAL
        assert fl.release([got[1], 10]) == slots.ERANGE
        assert fl.release([-1]) == slots.ERANGE
        assert fl.release([got[0], 12]) == slots.ERANGE          # range is checked first
        assert fl.order() == before and fl.available() == len(before)
        assert fl.alloc(-1)[0] == slots.EINVAL
        assert fl.release([got[1], got[2]]) == slots.OK          # the refused pages are still held


PINS = [pin_golden, pin_stamp_model, pin_partition, pin_lifo_reuses_last_batch,
        pin_churn_closed_forms, pin_refusals_change_nothing]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(slots.FreeList)


# ---- planted mistakes: each copy of the oracle differs in one step ------------------

class LifoReversed(slots.FreeList):
    def release(self, pages):
        rc = super().release(pages)
        if rc == slots.OK and self.policy == slots.LIFO and pages:
            n = len(pages)
            self.free[:n] = self.free[:n][::-1]
        return rc


class FifoAtHead(slots.FreeList):
    def release(self, pages):
        self.policy, saved = slots.LIFO, self.policy
        try:
            return super().release(pages)
        finally:
            self.policy = saved


class AllocFromTail(slots.FreeList):
    def alloc(self, k):
        if k < 0 or k > len(self.free):
            return super().alloc(k)
        taken = self.free[len(self.free) - k:][::-1] if k else []
        self.free = self.free[:len(self.free) - k]
        self.allocated.update(taken)
        return slots.OK, taken


class NoDuplicateCheck(slots.FreeList):
    def release(self, pages):
        pages = [int(p) for p in pages]
        if any(p < 0 or p >= self.num_pages for p in pages):
            return slots.ERANGE
        if any(p not in self.allocated for p in pages):
            return slots.EINVAL
        for p in set(pages):
            self.allocated.discard(p)
        self.free = self.free + pages if self.policy == slots.FIFO else pages + self.free
        return slots.OK


class StateBeforeRange(slots.FreeList):
    def release(self, pages):
        for p in pages:
            if 0 <= p < self.num_pages and p not in self.allocated:
                return slots.EINVAL
        return super().release(pages)


class PartialAlloc(slots.FreeList):
    def alloc(self, k):
        return super().alloc(min(k, len(self.free)))


class NoDoubleFreeCheck(slots.FreeList):
    def release(self, pages):
        pages = [int(p) for p in pages]
        if any(p < 0 or p >= self.num_pages for p in pages):
            return slots.ERANGE
        if len(set(pages)) != len(pages):
            return slots.EINVAL
        for p in pages:
            self.allocated.discard(p)
            if p in self.free:
                self.free.remove(p)
        self.free = self.free + pages if self.policy == slots.FIFO else pages + self.free
        return slots.OK


class OffByOneStart(slots.FreeList):
    def __init__(self, num_pages, policy):
        super().__init__(num_pages, policy)
        self.free = self.free[1:] + self.free[:1]


MUTANTS = [LifoReversed, FifoAtHead, AllocFromTail, NoDuplicateCheck, StateBeforeRange,
           PartialAlloc, NoDoubleFreeCheck, OffByOneStart]


def _fails_some_pin(cls):
    for pin in PINS:
        try:
            pin(cls)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(mutant):
    assert _fails_some_pin(mutant), mutant.__name__
