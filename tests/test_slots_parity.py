"""The library's host page allocator (kv_slots_*, include/kvslots.h) against
the free-list oracle (oracle/slots.py), operation by operation: allocated
pages, status codes and the whole free list after every call, on random
streams that mix valid calls with refused ones (too many pages, double frees,
pages listed twice, out-of-range pages). Host only: no GPU."""
import threading

import numpy as np
import pytest

from oracle import slots

POLICIES = (slots.FIFO, slots.LIFO)


@pytest.fixture(scope="module")
def kvt():
    import hierarchical_kv_cache_backup_amd as kvt
    return kvt


def mixed_stream(rng, P, steps):
    """Random operations; about a quarter of them are refused by both sides."""
    held = []
    for _ in range(steps):
        r = rng.random()
        if held and r < 0.45:
            m = int(rng.integers(1, len(held) + 1))
            pick = rng.permutation(len(held))[:m]
            batch = [held[j] for j in pick]
            yield "free", batch
            gone = set(batch)
            held = [h for h in held if h not in gone]
        elif r < 0.55:
            kind = int(rng.integers(0, 4))
            if kind == 0:
                batch = [int(rng.integers(P, P + 5))] if rng.random() < 0.5 else [-1]
            elif kind == 1 and held:
                batch = [held[0], held[0]]                      # listed twice
            else:
                free_now = sorted(set(range(P)) - set(held))
                batch = [free_now[0]] if free_now else [P]      # double free (or range)
            if held and rng.random() < 0.5:
                batch = [held[-1]] + batch
            yield "free", batch
        else:
            k = int(rng.integers(0, max(2, P // 3)))
            if rng.random() < 0.1:
                k = P - len(held) + 1                            # one too many
            got = yield "alloc", k
            held.extend(got or [])


def run_pair(kvt, P, policy, seed, steps, check_every=1):
    lib = kvt.HostPages(P, policy)
    ref = slots.FreeList(P, policy)
    gen = mixed_stream(np.random.default_rng(seed), P, steps)
    try:
        op, arg = next(gen)
        i = 0
        while True:
            if op == "alloc":
                rc, got = kvt.kv_slots_alloc(lib.handle, arg)
                rrc, rgot = ref.alloc(arg)
                assert rc == rrc, (P, policy, seed, i, op, arg)
                assert got.tolist() == rgot, (P, policy, seed, i, op, arg)
                nxt = gen.send(rgot if rrc == slots.OK else [])
            else:
                rc = kvt.kv_slots_free(lib.handle, arg)
                rrc = ref.release(arg)
                assert rc == rrc, (P, policy, seed, i, op, arg)
                nxt = next(gen)
            assert lib.available() == ref.available()
            if i % check_every == 0:
                assert lib.order().tolist() == ref.order(), (P, policy, seed, i)
            op, arg = nxt
            i += 1
    except StopIteration:
        pass
    assert lib.order().tolist() == ref.order()
    lib.close()


@pytest.mark.parametrize("policy", POLICIES, ids=["fifo", "lifo"])
def test_small_pools_every_operation(kvt, policy):
    for seed in range(40):
        P = int(np.random.default_rng([seed, 9]).integers(1, 40))
        run_pair(kvt, P, policy, seed, 120)


@pytest.mark.parametrize("policy", POLICIES, ids=["fifo", "lifo"])
def test_large_pool(kvt, policy):
    # a host pool of 65,536 pages (4M token slots at page size 64)
    run_pair(kvt, 65536, policy, 5, 400, check_every=50)


def test_argument_errors(kvt):
    assert kvt.kv_slots_create(0, 0)[0] == kvt.EINVAL
    assert kvt.kv_slots_create(-3, 0)[0] == kvt.EINVAL
    assert kvt.kv_slots_create(8, 2)[0] == kvt.EINVAL
    assert kvt.kv_slots_create((1 << 40) + 1, 0)[0] == kvt.EINVAL
    lib = kvt.library()
    assert lib.kv_slots_alloc(None, 1, None) == kvt.EINVAL
    assert lib.kv_slots_free(None, None, 0) == kvt.EINVAL
    assert lib.kv_slots_available(None) == kvt.EINVAL
    assert lib.kv_slots_destroy(None) == kvt.OK
    a = kvt.HostPages(4)
    assert lib.kv_slots_alloc(a.handle, -1, None) == kvt.EINVAL
    assert lib.kv_slots_alloc(a.handle, 2, None) == kvt.EINVAL
    assert lib.kv_slots_alloc(a.handle, 0, None) == kvt.OK
    assert lib.kv_slots_free(a.handle, None, 1) == kvt.EINVAL
    assert "null" in kvt.kv_last_error()
    assert lib.kv_slots_free(a.handle, None, -1) == kvt.EINVAL
    assert "n < 0" in kvt.kv_last_error()
    assert lib.kv_slots_free(a.handle, None, 0) == kvt.OK
    assert a.available() == 4
    with pytest.raises(kvt.KvError) as e:
        a.alloc(5)
    assert e.value.code == kvt.ENOMEM
    a.close()


def test_threads_partition_the_pool(kvt):
    """Four threads allocate and free at once; afterwards every page is either
    free once or held by exactly one thread."""
    P = 4096
    for policy in POLICIES:
        a = kvt.HostPages(P, policy)
        held = [[] for _ in range(4)]
        errors = []

        def worker(t):
            rng = np.random.default_rng(t)
            mine = held[t]
            try:
                for _ in range(3000):
                    if mine and rng.random() < 0.5:
                        m = int(rng.integers(1, len(mine) + 1))
                        a.free(mine[:m])
                        del mine[:m]
                    else:
                        rc, got = kvt.kv_slots_alloc(a.handle, int(rng.integers(1, 64)))
                        if rc == kvt.OK:
                            mine.extend(got.tolist())
                        elif rc != kvt.ENOMEM:
                            errors.append(rc)
            except Exception as ex:  # noqa: BLE001
                errors.append(ex)

        ts = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        assert not errors
        free = a.order().tolist()
        owned = [p for h in held for p in h]
        assert len(free) == len(set(free)) and len(owned) == len(set(owned))
        assert sorted(free + owned) == list(range(P))
        a.close()
