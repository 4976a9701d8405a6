"""The library-side serve loop (rt_serve_round + rt_prepare_extend_prio) and chunked prefill
(rt_chunk_launch + rt_prepare_extend) on the CPU: bit-exact with the oracle's scheduler (batch
picks, slot tables, final tree, free list), and on the hand-derived serve trace."""
import numpy as np
import pytest

import prefix_shared_kv_match_amd as pkv
from prefix_shared_kv_match_amd import runtime
from oracle import driver, scheduler
from oracle.radix_tree import OracleTree


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
