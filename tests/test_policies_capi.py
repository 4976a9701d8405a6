"""The library's eviction-policy family, read-only peek and cache-aware ordering on the CPU:
bit-exact with the oracle tree (node dump, per-node hit count / creation clock / priority,
eviction log, free list) for every policy, on random operation streams and on the multi-turn
workload's host side."""
import random

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import prefix_shared_kv_match_amd as pkv
from prefix_shared_kv_match_amd import runtime
from oracle import driver, scheduler
from oracle.radix_tree import POLICIES, OracleError, OracleTree


class Pair:
    def __init__(self, pool_slots, free_order, policy):
        self.o = OracleTree(pool_slots, free_order, policy)
        self.t = pkv.rt_create_policy(pool_slots, free_order, policy)

    def close(self):
        pkv.rt_destroy(self.t)

    def same(self):
        assert pkv.rt_dump(self.t) == self.o.dump()
        assert pkv.rt_dump_stats(self.t) == self.o.dump_stats()
        assert pkv.rt_copy_free_list(self.t).tolist() == list(self.o.free)
        assert pkv.rt_evictable_size(self.t) == self.o.evictable
        assert pkv.rt_protected_size(self.t) == self.o.protected
        assert pkv.rt_take_eviction_log(self.t) == [(i, list(s)) for i, s in self.o.take_evlog()]


def both(fo, fl):
    try:
        ro, eo = fo(), None
    except OracleError as e:
        ro, eo = None, e
    try:
        rl, el = fl(), None
    except pkv.PkvError as e:
        rl, el = None, e
    assert (eo is None) == (el is None), (eo, el)
    return ro, rl


def test_policy_codes_match_header_and_reject_unknown():
    assert sorted(pkv.RT_POLICIES) == sorted(POLICIES)
    import ctypes
    h = ctypes.c_void_p()
    with pytest.raises(pkv.PkvError):
        pkv.check(pkv.lib().rt_create_policy(8, None, 8, 7, ctypes.byref(h)))
    with pytest.raises(pkv.PkvError):
        pkv.check(pkv.lib().rt_create_policy(8, None, 8, -1, ctypes.byref(h)))


ops = st.lists(st.tuples(st.sampled_from(["prep", "prep", "match", "peek", "release", "evict", "alloc_free"]),
                         st.lists(st.integers(0, 3), min_size=0, max_size=9), st.integers(0, 12),
                         st.integers(0, 3)),
               min_size=1, max_size=40)


@pytest.mark.parametrize("policy", POLICIES)
@settings(max_examples=80, deadline=None)
@given(seq=ops, cap=st.integers(6, 40), seed=st.integers(0, 10_000))
def test_random_streams_match_oracle_per_policy(policy, seq, cap, seed):
    rng = random.Random(seed)
    pool = cap + rng.randrange(0, 5)
    order = rng.sample(range(pool), cap)
    P = Pair(pool, order, policy)
    held = []
    try:
        for op, toks, n, prio in seq:
            if op == "prep" and toks:
                ro, rl = both(lambda: driver.prepare_batch(P.o, [toks], [prio]),
                              lambda: runtime.prepare_prio(P.t, [np.array(toks)], 16, [prio]))
                if ro is not None:
                    assert rl.prefix_lens.tolist() == ro.prefix_lens
                    assert rl.req_to_token[0, :len(toks)].tolist() == ro.rows[0]
                    assert rl.last_nodes.tolist() == ro.last_nodes
                    held.append(ro.last_nodes[0])
            elif op == "match":
                ro, rl = both(lambda: P.o.match(toks), lambda: pkv.rt_match_prefix(P.t, toks))
                assert (ro[0], list(ro[1]), ro[2]) == (rl[0], rl[1].tolist(), rl[2])
            elif op == "peek":
                clock = pkv.rt_clock(P.t)
                assert pkv.rt_peek_prefix(P.t, toks) == P.o.peek(toks)
                assert pkv.rt_clock(P.t) == clock
            elif op == "release" and held:
                nid = held.pop(rng.randrange(len(held)))
                both(lambda: P.o.dec_lock(nid), lambda: pkv.rt_dec_lock_ref(P.t, nid))
            elif op == "evict":
                ro, rl = both(lambda: P.o.evict(n), lambda: pkv.rt_evict(P.t, n))
                assert ro == rl
            elif op == "alloc_free":
                ro, rl = both(lambda: P.o.alloc(n), lambda: pkv.rt_alloc(P.t, n))
                if ro is not None:
                    assert ro == rl.tolist()
                    both(lambda: P.o.free_slots(ro), lambda: pkv.rt_free(P.t, ro))
            P.same()
    finally:
        P.close()


def test_insert_priority_through_capi():
    P = Pair(32, None, "priority")
    try:
        s = pkv.rt_alloc(P.t, 5).tolist()
        assert P.o.alloc(5) == s
        assert P.o.insert([1, 2, 3, 4, 5], s, 3) == pkv.rt_insert_priority(P.t, [1, 2, 3, 4, 5], s, 3)
        s2 = pkv.rt_alloc(P.t, 2).tolist()
        assert P.o.alloc(2) == s2
        # walks [1, 2, 3] (split, upper inherits 3 and takes max(3, 7)) and hangs a new leaf
        assert P.o.insert([1, 2, 3, 9, 9], [-1, -1, -1] + s2, 7)[0] == \
            pkv.rt_insert_priority(P.t, [1, 2, 3, 9, 9], s[:3] + s2, 7)[0] == 3
        P.same()
        stats = {nid: prio for nid, _, _, prio in pkv.rt_dump_stats(P.t)}
        assert sorted(stats.values()) == [3, 7, 7]
    finally:
        P.close()


@pytest.mark.parametrize("policy", POLICIES)
def test_multiturn_host_bit_exact_per_policy(policy):
    import workloads
    wl = workloads.multiturn_bf16(n_conv=96, capacity=160_000)
    ob = driver.run_workload_host(wl, policy=policy)
    lb, ldec, levlog, lfree, lev, lprot, ldump = runtime.run_workload_host(wl, policy=policy)
    for o, l in zip(ob.batches, lb):
        assert l.prefix_lens.tolist() == o.prefix_lens
        assert l.new_slots.tolist() == o.new_slots
        assert l.last_nodes.tolist() == o.last_nodes
    assert levlog == [(i, list(s)) for i, s in ob.evlog]
    assert lfree == ob.free and ldump == ob.dump
    assert len(ob.evlog) > 0


@settings(max_examples=60, deadline=None)
@given(reqs=st.lists(st.lists(st.integers(0, 3), min_size=0, max_size=8), min_size=0, max_size=12),
       cached=st.lists(st.lists(st.integers(0, 3), min_size=1, max_size=8), min_size=0, max_size=5))
def test_schedule_longest_prefix_matches_oracle_order(reqs, cached):
    P = Pair(128, None, "lru")
    try:
        for c in cached:
            driver.release(P.o, driver.prepare_batch(P.o, [c]).last_nodes)
            pkv.rt_release(P.t, runtime.prepare(P.t, [np.array(c)], 16).last_nodes)
        toks, indptr = runtime.flatten([np.array(r, dtype=np.int32) for r in reqs])
        order, lens = pkv.rt_schedule_longest_prefix(P.t, toks, indptr)
        assert order.tolist() == scheduler.schedule_order(P.o, reqs, "lpm")
        assert lens.tolist() == [P.o.peek(r) for r in reqs]
        P.same()
    finally:
        P.close()
