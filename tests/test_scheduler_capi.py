"""The library-side serve loop (rt_serve_round + rt_prepare_extend_prio) and chunked prefill
(rt_chunk_prepare + rt_chunk_finish) on the CPU: bit-exact with the oracle's scheduler (batch
picks, slot tables, final tree, free list), and on the hand-derived serve trace."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import prefix_shared_kv_match_amd as pkv
from prefix_shared_kv_match_amd import runtime
from oracle import driver, scheduler
from oracle.radix_tree import OOMError, OracleTree


def same_tree(t, o):
    assert pkv.rt_dump(t) == o.dump()
    assert pkv.rt_dump_stats(t) == o.dump_stats()
    assert pkv.rt_copy_free_list(t).tolist() == list(o.free)
    assert pkv.rt_take_eviction_log(t) == [(i, list(s)) for i, s in o.take_evlog()]


@pytest.mark.parametrize("order,policy", [("fcfs", "lru"), ("lpm", "lru"), ("lpm", "lfu"), ("fcfs", "priority"),
                                          ("lpm", "slru")])
def test_serve_matches_oracle(order, policy):
    import workloads
    wl = workloads.multiturn_bf16(n_conv=64, capacity=120_000)
    arr = [r for b in wl.batches for r in b]
    after = [r.after for r in arr]
    prio = [r.priority for r in arr]
    o = OracleTree(wl.pool_slots, wl.free_order, policy)
    log = scheduler.serve(o, [r.tokens.tolist() for r in arr], after, order, batch=16, window=64, priorities=prio)
    t = pkv.rt_create_policy(wl.pool_slots, wl.free_order, policy)
    try:
        seen = []
        out = runtime.serve(t, [r.tokens for r in arr], after, order, 16, 64, wl.max_len(), priorities=prio,
                            on_batch=lambda pick, hb: seen.append(len(pick)))
        assert [p for p, _ in out] == log.picks
        assert seen == [len(p) for p in log.picks]
        for (pick, hb), bt in zip(out, log.tables):
            assert hb.prefix_lens.tolist() == bt.prefix_lens
            assert hb.new_slots.tolist() == bt.new_slots
            for i, row in enumerate(bt.rows):
                assert hb.req_to_token[i, :len(row)].tolist() == row
        same_tree(t, o)
    finally:
        pkv.rt_destroy(t)


def test_serve_rejects_bad_arguments():
    t = pkv.rt_create(16)
    try:
        with pytest.raises(ValueError):
            runtime.serve(t, [np.array([1])], [-1], "random", 1, 1, 4)
        with pytest.raises(pkv.PkvError, match="bad arguments"):
            runtime.serve(t, [np.array([1])], [-1], "fcfs", 0, 1, 4)
        with pytest.raises(pkv.PkvError, match="not earlier"):      # a dependency that points forward
            runtime.serve(t, [np.array([1]), np.array([2])], [1, -1], "fcfs", 1, 1, 4)
    finally:
        pkv.rt_destroy(t)


@pytest.mark.parametrize("budget", [1, 5, 33, 200, 10**6])
def test_chunked_prefill_matches_oracle(budget):
    import workloads
    wl = workloads.fewshot_bf16(n_req=6, prefix_len=90, suffix_range=(20, 60))
    reqs = [r.tokens for r in wl.batches[0]] + [wl.batches[0][0].tokens[:50]]   # one fully cached request
    o = OracleTree(wl.pool_slots, wl.free_order)
    t = pkv.rt_create(wl.pool_slots, wl.free_order)
    try:
        for r in wl.pre_insert:
            driver.release(o, driver.prepare_batch(o, [r.tokens]).last_nodes)
            pkv.rt_release(t, runtime.prepare(t, [r.tokens], 256).last_nodes)
        ls = scheduler.chunked_prefill(o, [x.tolist() for x in reqs], budget)
        got = runtime.chunked_prefill(t, reqs, budget, 256)
        assert [(r_, e_) for r_, e_, _ in got] == [(l.reqs, l.ends) for l in ls]
        for (_, _, hb), l in zip(got, ls):
            assert hb.prefix_lens.tolist() == l.tables.prefix_lens
            assert hb.extend_lens.tolist() == l.tables.extend_lens
            assert hb.new_slots.tolist() == l.tables.new_slots
        same_tree(t, o)
        assert pkv.rt_protected_size(t) == 0
    finally:
        pkv.rt_destroy(t)


@settings(max_examples=120, deadline=None)
@given(st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=12), min_size=1, max_size=6),
       st.integers(1, 20), st.lists(st.integers(0, 2), max_size=8), st.integers(12, 60))
def test_chunked_prefill_random_matches_oracle(reqs, budget, cached, slots):
    """Random small batches (vocab 3, so requests share and split nodes), a random cached
    prefix, budgets from one token up and pools small enough that launches evict: the
    library's launches (rt_chunk_prepare / rt_chunk_finish) equal the oracle's, launch for
    launch (cut, prefix and extend lengths, new slots), and the final trees match."""
    o = OracleTree(slots)
    t = pkv.rt_create(slots)
    try:
        if cached:
            driver.release(o, driver.prepare_batch(o, [cached]).last_nodes)
            pkv.rt_release(t, runtime.prepare(t, [np.array(cached)], 16).last_nodes)
        try:
            ls = scheduler.chunked_prefill(o, reqs, budget)
        except OOMError:   # both sides run out of slots (in the same launch)
            with pytest.raises(pkv.PkvError):
                runtime.chunked_prefill(t, [np.array(r) for r in reqs], budget, 16)
            return
        got = runtime.chunked_prefill(t, [np.array(r) for r in reqs], budget, 16)
        assert [(r_, e_) for r_, e_, _ in got] == [(l.reqs, l.ends) for l in ls]
        for (_, _, hb), l in zip(got, ls):
            assert hb.prefix_lens.tolist() == l.tables.prefix_lens
            assert hb.extend_lens.tolist() == l.tables.extend_lens
            assert hb.new_slots.tolist() == l.tables.new_slots
        same_tree(t, o)
        assert pkv.rt_protected_size(t) == 0
    finally:
        pkv.rt_destroy(t)


def test_chunk_prepare_and_finish_hand_example():
    """rt_chunk_prepare / rt_chunk_finish on the two-launch example: budget 4, r0 = [1..6],
    r1 = [1, 2, 3, 9], nothing cached.  Launch 1 takes r0 to 4 and leaves r0's end node
    locked (4 protected tokens); launch 2 continues r0 to 6 and takes r1's 1 new token after
    its 3 cached ones, moving r0's lock to its new end node before the old one is dropped;
    the finish unlocks both finished requests and the head passes them."""
    t = pkv.rt_create(32)
    try:
        toks, indptr = runtime.flatten([np.arange(1, 7), np.array([1, 2, 3, 9])])
        done = np.full(2, -1, dtype=np.int64)
        held = np.full(2, -1, dtype=np.int64)
        r2t = np.full((2, 8), -1, dtype=np.int32)
        reqs, ends, pl, el, qo, new = pkv.rt_chunk_prepare(t, toks, indptr, done, held, 0, 4, r2t)
        assert reqs.tolist() == [0] and ends.tolist() == [4]
        assert pl.tolist() == [0] and el.tolist() == [4] and qo.tolist() == [0, 4] and new.size == 4
        assert done.tolist() == [4, -1] and held[0] >= 0 and held[1] == -1
        first_rows = r2t[0, :4].copy()
        assert pkv.rt_protected_size(t) == 4
        assert pkv.rt_chunk_finish(t, indptr, reqs, done, held, 0) == 0      # r0 not finished: still held
        assert pkv.rt_protected_size(t) == 4
        old = int(held[0])
        r2t[:] = -1
        reqs, ends, pl, el, qo, new = pkv.rt_chunk_prepare(t, toks, indptr, done, held, 0, 4, r2t)
        assert reqs.tolist() == [0, 1] and ends.tolist() == [6, 4]
        assert pl.tolist() == [4, 3] and el.tolist() == [2, 1] and qo.tolist() == [0, 2, 3]
        assert r2t[0, :4].tolist() == first_rows.tolist() and r2t[1, :3].tolist() == first_rows[:3].tolist()
        assert held[0] != old and done.tolist() == [6, 4]
        # lock_ref per node key: r0's path [1,2,3]-[4]-[5,6] and r1's [1,2,3]-[9] hold one
        # lock each; a first-chunk lock left behind would put 3 on [1,2,3] and 2 on [4]
        locks = {key: lock for _, _, lock, _, key, _ in pkv.rt_dump(t)}
        assert locks == {(1, 2, 3): 2, (4,): 1, (5, 6): 1, (9,): 1}
        assert pkv.rt_chunk_finish(t, indptr, reqs, done, held, 0) == 2
        assert held.tolist() == [-1, -1] and pkv.rt_protected_size(t) == 0
        assert pkv.rt_evictable_size(t) == 7
        with pytest.raises(pkv.PkvError):
            pkv.rt_chunk_finish(t, indptr, np.array([2], dtype=np.int32), done, held, 0)   # no request 2
    finally:
        pkv.rt_destroy(t)


def test_chunk_prepare_failure_leaves_state():
    """A launch whose prepare runs out of slots fails, leaves done / held as they were and
    leaves no lock behind: a 6-slot pool, r0 = 4 tokens held from a first launch, then a
    launch needing 4 more tokens (2 for r0, 2 for a new r1) while only 2 slots are free."""
    t = pkv.rt_create(6)
    try:
        toks, indptr = runtime.flatten([np.arange(1, 7), np.array([7, 8])])
        done = np.full(2, -1, dtype=np.int64)
        held = np.full(2, -1, dtype=np.int64)
        r2t = np.full((2, 8), -1, dtype=np.int32)
        pkv.rt_chunk_prepare(t, toks, indptr, done, held, 0, 4, r2t)
        state = (done.copy(), held.copy())
        with pytest.raises(pkv.PkvError):
            pkv.rt_chunk_prepare(t, toks, indptr, done, held, 0, 8, r2t)
        assert done.tolist() == state[0].tolist() and held.tolist() == state[1].tolist()
        assert pkv.rt_protected_size(t) == 4        # only r0's first chunk, as before the call
    finally:
        pkv.rt_destroy(t)


def test_chunk_launch_hand_example():
    """rt_chunk_launch, the cut of one chunked-prefill launch: [1,2,3] cached; requests
    [1,2,3,4,5] (2 uncached tokens) and [9,9,9] (3) under a budget of 4 -> the first takes its
    2 tokens (end 5), the second 2 of its 3 (end 2, cut); the next launch from the cut request
    (2 done) takes its last token (end 3).  The tree is not changed."""
    t = pkv.rt_create(32)
    try:
        hb = runtime.prepare(t, [np.array([1, 2, 3])], 8)
        pkv.rt_release(t, hb.last_nodes)
        before = (pkv.rt_dump(t), pkv.rt_clock(t))
        toks, indptr = runtime.flatten([np.array([1, 2, 3, 4, 5]), np.array([9, 9, 9])])
        reqs, ends = pkv.rt_chunk_launch(t, toks, indptr, [-1, -1], 0, 4)
        assert reqs.tolist() == [0, 1] and ends.tolist() == [5, 2]
        reqs, ends = pkv.rt_chunk_launch(t, toks, indptr, [5, 2], 1, 4)
        assert reqs.tolist() == [1] and ends.tolist() == [3]
        assert (pkv.rt_dump(t), pkv.rt_clock(t)) == before
        with pytest.raises(pkv.PkvError):
            pkv.rt_chunk_launch(t, toks, indptr, [-1, -1], 0, 0)       # no budget
        with pytest.raises(pkv.PkvError):
            pkv.rt_chunk_launch(t, toks, indptr, [9, -1], 0, 4)       # more done than the request holds
    finally:
        pkv.rt_destroy(t)


def _hand():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "serve_window_dependency.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _hand()["cases"], ids=lambda c: f"w{c['window']}-{c['order']}-n{c['n']}")
def test_serve_rounds_hand_example(case):
    """The library's rounds (rt_serve_round) on the hand-derived serve trace
    (tests/golden/serve_window_dependency.json) the oracle's serve loop is pinned to."""
    g = _hand()
    n = case["n"]
    t = pkv.rt_create(64)
    try:
        hb = runtime.prepare_prio(t, [np.array(g["cached"])], 16, None)
        pkv.rt_release(t, hb.last_nodes)
        got = runtime.serve(t, [np.array(r) for r in g["requests"][:n]], g["after"][:n], case["order"], g["batch"],
                            case["window"], 16)
        assert [p for p, _ in got] == case["picks"]
        by_req = {}
        for p, hb in got:
            for i, r in enumerate(p):
                by_req[r] = int(hb.prefix_lens[i])
        assert [by_req[r] for r in range(n)] == case["prefix_by_request"]
    finally:
        pkv.rt_destroy(t)
