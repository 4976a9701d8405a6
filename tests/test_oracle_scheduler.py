"""Pins for the oracle's serve loop (cache-aware scheduling) and chunked prefill.

- With a window of one batch, no dependencies and FCFS the serve loop reduces to the plain
  batch driver over consecutive arrivals (itself pinned by the worked examples).
- Two hand-derived traces on a 12-slot pool (derivations in the test bodies) fix the
  longest-prefix-first order, its eviction interplay and the chunk cut points.
- A hand-derived serve trace (tests/golden/serve_window_dependency.json) fixes the waiting
  window, a dependency and the tie rule in both orders.
- Invariants on the multi-turn workload: every request is served once, never before the
  request it depends on, batches stay within size, and LPM's order is a valid sort.
"""
import pytest

from oracle import driver, scheduler
from oracle.radix_tree import OracleError, OracleTree


def test_fcfs_one_window_reduces_to_plain_batches():
    import workloads
    wl = workloads.multiturn_bf16(n_conv=64, capacity=150_000)
    arrivals = [r for b in wl.batches for r in b]
    toks = [r.tokens.tolist() for r in arrivals]
    t = OracleTree(wl.pool_slots, wl.free_order)
    log = scheduler.serve(t, toks, [-1] * len(toks), "fcfs", batch=32, window=32)
    ref = driver.run_workload_host(wl)
    assert [len(p) for p in log.picks] == [len(b) for b in wl.batches]
    assert log.picks[0] == list(range(32))
    for a, b in zip(log.tables, ref.batches):
        assert a.rows == b.rows and a.prefix_lens == b.prefix_lens and a.new_slots == b.new_slots
    assert t.dump() == ref.dump and list(t.free) == ref.free


P = list(range(100, 110))      # a 10-token prefix
Q = list(range(200, 210))      # another one


def test_lpm_beats_fcfs_on_hand_trace():
    """12-slot pool (identity free order), one request per batch, window 4.

    r0 = P+[1], r1 = Q+[2], r2 = P+[3], r3 = Q+[4] (11 tokens each).
    FCFS: each request needs 11 of the 12 slots, so it evicts its predecessor's leaf
    (the only unlocked leaf) before a prefix can be reused: 0 cached tokens.
    LPM: round 1 peeks are all 0, r0 goes first; round 2 peeks r1=0, r2=10, r3=0 so r2
    runs (split P|[1], one new slot); round 3 peeks r1=0, r3=0 so r1 runs and evicts
    [1], [3] then P (12 tokens for an 11-token shortfall); round 4 r3 reuses Q: 20 cached."""
    reqs = [P + [1], Q + [2], P + [3], Q + [4]]
    fc = scheduler.serve(OracleTree(12), reqs, [-1] * 4, "fcfs", batch=1, window=4)
    assert fc.picks == [[0], [1], [2], [3]]
    assert [b.prefix_lens for b in fc.tables] == [[0], [0], [0], [0]]
    assert fc.cached_tokens == 0 and fc.prompt_tokens == 44
    t = OracleTree(12)
    lp = scheduler.serve(t, reqs, [-1] * 4, "lpm", batch=1, window=4)
    assert lp.picks == [[0], [2], [1], [3]]
    assert [b.prefix_lens for b in lp.tables] == [[0], [10], [0], [10]]
    assert lp.cached_tokens == 20
    # round 3 evicts r0's split-off [1] (node 1, slot 10), r2's leaf [3] (node 3, slot 11) and
    # then P (node 2, slots 0..9), in that (access time, id) order
    assert t.take_evlog() == [(1, [10]), (3, [11]), (2, list(range(10)))]


def test_lpm_order_and_ties():
    t = OracleTree(64)
    for key in (P[:4], Q[:2]):
        driver.release(t, driver.prepare_batch(t, [key]).last_nodes)
    reqs = [[7, 8], Q[:2] + [9], P[:4] + [0], P[:2] + [9], [7]]
    assert scheduler.schedule_order(t, reqs, "lpm") == [2, 1, 3, 0, 4]
    assert scheduler.schedule_order(t, reqs, "fcfs") == [0, 1, 2, 3, 4]
    clock = t.clock
    scheduler.schedule_order(t, reqs, "lpm")
    assert t.clock == clock                      # ordering reads the tree only
    with pytest.raises(OracleError):
        scheduler.schedule_order(t, reqs, "random")


def _serve_hand():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "serve_window_dependency.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _serve_hand()["cases"], ids=lambda c: f"w{c['window']}-{c['order']}-n{c['n']}")
def test_serve_window_and_dependency_hand_trace(case):
    """Serve rounds under a waiting window, a dependency (r2 waits for r0) and a tie of cached
    prefix lengths, in both orders, against the hand derivation in the fixture."""
    g = _serve_hand()
    n = case["n"]
    t = OracleTree(64)
    bt = driver.prepare_batch(t, [g["cached"]])
    driver.release(t, bt.last_nodes)
    log = scheduler.serve(t, g["requests"][:n], g["after"][:n], case["order"], g["batch"], case["window"])
    assert log.picks == case["picks"]
    by_req = {}
    for pick, tab in zip(log.picks, log.tables):
        for r, pl in zip(pick, tab.prefix_lens):
            by_req[r] = pl
    assert [by_req[r] for r in range(n)] == case["prefix_by_request"]


@pytest.mark.parametrize("order", scheduler.ORDERS)
def test_serve_invariants_on_multiturn(order):
    import workloads
    wl = workloads.multiturn_bf16(n_conv=64, capacity=150_000)
    arrivals = [r for b in wl.batches for r in b]
    toks = [r.tokens.tolist() for r in arrivals]
    after = [r.after for r in arrivals]
    assert any(a >= 0 for a in after)
    log = scheduler.serve(OracleTree(wl.pool_slots, wl.free_order), toks, after, order, batch=16, window=64)
    round_of = {}
    for k, pick in enumerate(log.picks):
        assert 1 <= len(pick) <= 16
        for i in pick:
            assert i not in round_of
            round_of[i] = k
    assert sorted(round_of) == list(range(len(toks)))
    for i, a in enumerate(after):
        if a >= 0:
            assert round_of[a] < round_of[i]
    assert log.prompt_tokens == sum(len(x) for x in toks)
    assert 0 < log.cached_tokens < log.prompt_tokens


def test_chunked_prefill_hand_trace():
    """Budget 4.  r0 = [1..6] (nothing cached), r1 = [1, 2, 3, 9].
    Launch 1: r0 takes 4 tokens (ends at 4); the budget is spent.
    Launch 2: r0 goes on from 4 and takes its last 2; r1 peeks 3 ([1, 2, 3] is cached by
    r0's first chunk) and takes its 1 new token.  Prefix lengths [0] then [4, 3]."""
    t = OracleTree(32)
    ls = scheduler.chunked_prefill(t, [[1, 2, 3, 4, 5, 6], [1, 2, 3, 9]], 4)
    assert [(l.reqs, l.ends) for l in ls] == [([0], [4]), ([0, 1], [6, 4])]
    assert [l.tables.prefix_lens for l in ls] == [[0], [4, 3]]
    assert [l.tables.extend_lens for l in ls] == [[4], [2, 1]]
    assert ls[1].tables.rows[0][:4] == ls[0].tables.rows[0]
    assert t.protected == 0 and t.evictable == 7


def test_chunked_prefill_large_budget_is_plain_prepare():
    import workloads
    wl = workloads.fewshot_bf16(n_req=8, prefix_len=120, suffix_range=(10, 30))
    toks = [r.tokens.tolist() for r in wl.batches[0]]
    a = OracleTree(wl.pool_slots, wl.free_order)
    for r in wl.pre_insert:
        driver.release(a, driver.prepare_batch(a, [r.tokens]).last_nodes)
    b = OracleTree(wl.pool_slots, wl.free_order)
    for r in wl.pre_insert:
        driver.release(b, driver.prepare_batch(b, [r.tokens]).last_nodes)
    ls = scheduler.chunked_prefill(a, toks, 10**9)
    bt = driver.prepare_batch(b, toks)
    driver.release(b, bt.last_nodes)
    assert len(ls) == 1 and ls[0].tables.rows == bt.rows and ls[0].tables.prefix_lens == bt.prefix_lens
    assert a.dump() == b.dump()


@pytest.mark.parametrize("budget", [1, 7, 64, 300])
def test_chunked_prefill_invariants(budget):
    import workloads
    wl = workloads.fewshot_bf16(n_req=6, prefix_len=90, suffix_range=(20, 60))
    toks = [r.tokens.tolist() for r in wl.batches[0]]
    t = OracleTree(wl.pool_slots, wl.free_order)
    for r in wl.pre_insert:
        driver.release(t, driver.prepare_batch(t, [r.tokens]).last_nodes)
    first = [t.peek(x) for x in toks]
    ls = scheduler.chunked_prefill(t, toks, budget)
    covered = {i: [] for i in range(len(toks))}
    for l in ls:
        assert sum(l.tables.extend_lens) <= budget
        for i, e, pl, el in zip(l.reqs, l.ends, l.tables.prefix_lens, l.tables.extend_lens):
            assert pl + el == e
            covered[i].append((pl, e))
    for i, spans in covered.items():
        assert spans[0][0] >= first[i] or spans[0][0] == spans[0][1]
        assert spans[-1][1] == len(toks[i])
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert b0 == a1
    assert t.protected == 0
    for x in toks:                                # every request ends up cached in full
        assert t.peek(x) == len(x)
