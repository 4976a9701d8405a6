"""Pins for the oracle radix tree: printed worked example, split picture, derived eviction
order, a brute-force longest-common-prefix model, and lock/evict/slot invariants."""
import heapq
import json
import os
import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle import driver
from oracle.radix_tree import LockError, NodeError, OOMError, OracleTree, SlotError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def build(inserts, pool_slots):
    t = OracleTree(pool_slots)
    for toks in inserts:
        bt = driver.prepare_batch(t, [toks])
        driver.release(t, bt.last_nodes)
    return t


def nodes_by_path(t):
    out = {}
    for nid, par, lock, last, key, val in t.dump():
        out[tuple(t.path_tokens(nid))] = (key, val, lock)
    return out


def test_worked_example_tree_and_hit():
    g = load("radix_worked_example.json")
    t = build(g["inserts"], g["pool_slots"])
    assert t.root.lock_ref == g["root_lock_ref"]
    byp = nodes_by_path(t)
    assert len(byp) == len(g["tree"])
    for n in g["tree"]:
        key, val, lock = byp[tuple(n["path"])]
        assert list(key) == n["key"]
        assert list(val) == n["kv"]
        assert lock == 0
    m, slots, _ = t.match(g["query"])
    assert m == g["match_len"]
    assert slots == g["match_slots"]


def test_split_example():
    g = load("radix_split_example.json")
    t = OracleTree(16)
    key = g["before"]["key"]
    bt = driver.prepare_batch(t, [key])          # leaf [1..5], locked
    (leaf,) = bt.last_nodes
    m, slots, upper = t.match(key[: g["split_len"]])
    assert m == g["split_len"] and slots == bt.rows[0][: g["split_len"]]
    d = {nid: (par, lock, k, v) for nid, par, lock, _, k, v in t.dump()}
    assert list(d[upper][2]) == g["after_upper"]["key"]
    assert list(d[leaf][2]) == g["after_lower"]["key"]
    assert d[leaf][0] == upper and d[upper][0] == 0
    # the upper node inherits the lock reference; counts move with the tokens
    assert d[upper][1] == d[leaf][1] == 1
    assert t.protected == 5 and t.evictable == 0
    driver.release(t, [leaf])
    assert t.protected == 0 and t.evictable == 5


def test_derived_eviction_order():
    g = load("radix_worked_example.json")
    e = load("eviction_derived.json")
    t = build(g["inserts"], g["pool_slots"])
    bt = driver.prepare_batch(t, [e["extra_insert"]])
    assert bt.rows[0][-1] == e["extra_slot"]
    driver.release(t, bt.last_nodes)
    for call in e["evict_calls"]:
        n = t.evict(call["num_tokens"])
        log = t.take_evlog()
        assert n == call["evicted"]
        assert [list(s) for _, s in log] == call["freed"]


def test_locked_path_is_never_evicted_and_oom():
    t = OracleTree(8)
    bt = driver.prepare_batch(t, [[1, 2, 3, 4, 5, 6]])   # 6 slots, locked
    with pytest.raises(OOMError):
        t.alloc(3)
    assert t.take_evlog() == []
    driver.release(t, bt.last_nodes)
    got = t.alloc(3)                                       # evicts the whole 6-token leaf
    assert len(got) == 3
    assert [len(s) for _, s in t.take_evlog()] == [6]


def test_error_paths():
    t = OracleTree(4)
    with pytest.raises(LockError):
        bt = driver.prepare_batch(t, [[1, 2]])
        driver.release(t, bt.last_nodes)
        driver.release(t, bt.last_nodes)
    with pytest.raises(SlotError):
        t.free_slots([2])                                  # slot 2 is free already
    with pytest.raises(SlotError):
        t.free_slots([99])
    with pytest.raises(NodeError):
        t.inc_lock(12345)
    with pytest.raises(SlotError):
        OracleTree(4, [0, 0, 1])


def check_invariants(t: OracleTree, in_flight: int = 0):
    dump = t.dump()
    total = sum(len(k) for _, _, _, _, k, _ in dump)
    prot = sum(len(k) for _, _, lock, _, k, _ in dump if lock > 0)
    assert t.evictable + t.protected == total
    assert t.protected == prot
    locks = {nid: lock for nid, _, lock, _, _, _ in dump}
    for nid, par, lock, _, key, val in dump:
        assert len(key) == len(val) > 0
        if par != 0:
            assert locks[par] >= lock
    cached = [s for *_, v in dump for s in v]
    assert len(set(cached)) == len(cached)
    assert not set(cached) & set(t.free)
    assert len(t.free) + len(cached) + in_flight == t.capacity


def brute_match(model, toks):
    m = 0
    while m < len(toks) and tuple(toks[: m + 1]) in model:
        m += 1
    return m, [model[tuple(toks[: j + 1])] for j in range(m)]


def run_against_brute_force(seqs, capacity, release_pattern, seed):
    """Drive the oracle with the per-request driver and check every match against a dict of
    cached token prefixes (prefix tuple -> slot of its last token), updated from the eviction log."""
    rng = random.Random(seed)
    t = OracleTree(capacity, list(rng.sample(range(capacity), capacity)))
    model = {}
    held = []
    for i, toks in enumerate(seqs):
        exp_m, exp_slots = brute_match(model, toks)
        assert t.peek(toks) == exp_m
        try:
            bt = driver.prepare_batch(t, [toks])
        except OOMError:
            # everything else is locked; release the oldest holder and go on
            for _, s in t.take_evlog():
                gone = [p for p, sl in model.items() if sl in set(s)]
                assert len(gone) == len(s)
                for p in gone:
                    del model[p]
            if held:
                driver.release(t, [held.pop(0)])
            check_invariants(t)
            continue
        assert bt.prefix_lens[0] == exp_m, (i, toks)
        assert bt.rows[0][:exp_m] == exp_slots
        for nid, slots in t.take_evlog():
            s = set(slots)
            gone = [p for p, sl in model.items() if sl in s]
            assert len(gone) == len(slots)
            for p in gone:
                del model[p]
        for j in range(len(toks)):
            model[tuple(toks[: j + 1])] = bt.rows[0][j]
        # the cached set stays prefix closed and equals the tree's slots
        for p in model:
            assert len(p) == 1 or p[:-1] in model
        assert sorted(model.values()) == sorted(s for *_, v in t.dump() for s in v)
        held.append(bt.last_nodes[0])
        while held and release_pattern[i % len(release_pattern)] and len(held) > 0:
            driver.release(t, [held.pop(0)])
            break
        check_invariants(t)
    for n in held:
        driver.release(t, [n])
    check_invariants(t)


seq_strategy = st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=10), min_size=1, max_size=12)


@settings(max_examples=300, deadline=None)
@given(seqs=seq_strategy, capacity=st.integers(10, 40),
       release_pattern=st.lists(st.booleans(), min_size=1, max_size=4), seed=st.integers(0, 1000))
def test_brute_force_lcp(seqs, capacity, release_pattern, seed):
    run_against_brute_force(seqs, capacity, release_pattern, seed)


def test_brute_force_lcp_long_run():
    rng = random.Random(7)
    seqs = [[rng.randrange(3) for _ in range(rng.randrange(1, 12))] for _ in range(400)]
    run_against_brute_force(seqs, 30, [True, False, True], 3)


def brute_evict(dump, n):
    """Expected eviction from a snapshot: repeatedly drop the min (last, id) unlocked childless node."""
    nodes = {nid: dict(par=par, lock=lock, last=last, val=list(v)) for nid, par, lock, last, _, v in dump}
    out = []
    got = 0
    while got < n:
        parents = {x["par"] for x in nodes.values()}
        cands = [(x["last"], nid) for nid, x in nodes.items() if x["lock"] == 0 and nid not in parents]
        if not cands:
            break
        _, nid = min(cands)
        out.append((nid, nodes[nid]["val"]))
        got += len(nodes[nid]["val"])
        del nodes[nid]
    return out


@settings(max_examples=200, deadline=None)
@given(seqs=seq_strategy, n=st.integers(1, 30), seed=st.integers(0, 1000), keep=st.integers(0, 3))
def test_eviction_order_matches_brute_force(seqs, n, seed, keep):
    rng = random.Random(seed)
    t = OracleTree(200, list(rng.sample(range(200), 200)))
    held = []
    for toks in seqs:
        bt = driver.prepare_batch(t, [toks])
        held.append(bt.last_nodes[0])
    for nid in held[keep:]:
        driver.release(t, [nid])
    expect = brute_evict(t.dump(), n)
    t.evict(n)
    assert [(nid, list(s)) for nid, s in t.take_evlog()] == expect
    check_invariants(t)


def test_clock_stamps_every_visited_node():
    t = OracleTree(64)
    for toks in ([1, 2, 3, 4], [1, 2, 9], [1, 2, 3, 7]):
        driver.release(t, driver.prepare_batch(t, [toks]).last_nodes)
    c0 = t.clock
    t.match([1, 2, 3, 4, 5])
    lasts = {tuple(t.path_tokens(nid)): last for nid, _, _, last, _, _ in t.dump()}
    assert lasts[(1, 2)] == c0 + 1 and lasts[(1, 2, 3)] == c0 + 1 and lasts[(1, 2, 3, 4)] == c0 + 1
    assert lasts[(1, 2, 9)] < c0 + 1 and lasts[(1, 2, 3, 7)] < c0 + 1


def test_insert_splits_partial_node():
    t = OracleTree(64)
    t.insert([1, 2, 3, 4], [10, 11, 12, 13])
    total, end = t.insert([1, 2, 5], [10, 11, 20])
    assert total == 2
    byp = nodes_by_path(t)
    assert byp[(1, 2)][0] == (1, 2) and byp[(1, 2, 3, 4)][0] == (3, 4) and byp[(1, 2, 5)][0] == (5,)
    # a key that ends inside a node splits it too, and returns the upper node
    total, end = t.insert([1, 2, 3], [10, 11, 12])
    assert total == 3 and tuple(t.path_tokens(end)) == (1, 2, 3)
    assert t.evictable == 5


def test_free_list_is_fifo():
    # identity order: slots 0..12 handed out in order; evicted slots go to the tail, so the
    # next allocation takes the head (13), and the evicted ones come back in eviction order
    g = load("radix_worked_example.json")
    t = build(g["inserts"], 16)                  # 12 of 16 slots used
    driver.release(t, driver.prepare_batch(t, [[1, 2, 3, 4, 5, 6]]).last_nodes)   # slot 12
    t.evict(1)                                    # frees [5, 6] to the tail
    assert t.alloc(1) == [13]
    assert t.alloc(4) == [14, 15, 5, 6]


def test_insert_stamps_visited_nodes():
    t = OracleTree(64)
    t.insert([1, 2, 3, 4], [10, 11, 12, 13])
    t.insert([1, 2, 5], [10, 11, 20])
    c = t.clock
    t.insert([1, 2, 3, 4, 9], [10, 11, 12, 13, 30])
    lasts = {tuple(t.path_tokens(nid)): last for nid, _, _, last, _, _ in t.dump()}
    assert lasts[(1, 2)] == lasts[(1, 2, 3, 4)] == lasts[(1, 2, 3, 4, 9)] == c + 1
    assert lasts[(1, 2, 5)] == c


# ---------------------------------------------------------------------------------------------
# eviction-policy family and the read-only peek (the radix-cache page's strategy list; the
# keys are readings documented in the oracle's module docstring)
# ---------------------------------------------------------------------------------------------

from oracle.radix_tree import POLICIES, evict_key  # noqa: E402


def brute_evict_policy(t, n):
    """Expected eviction from a snapshot under t.policy: repeatedly drop the unlocked childless
    node with the smallest policy key (keys recomputed from the dumped fields)."""
    stats = {nid: (h, c, p) for nid, h, c, p in t.dump_stats()}
    nodes = {}
    for nid, par, lock, last, _, v in t.dump():
        h, c, p = stats[nid]
        nodes[nid] = dict(par=par, lock=lock, val=list(v), key=None, last=last, hits=h, created=c, priority=p)

    class N:
        pass
    out, got = [], 0
    while got < n:
        parents = {x["par"] for x in nodes.values()}
        cands = []
        for nid, x in nodes.items():
            if x["lock"] or nid in parents:
                continue
            o = N()
            o.id, o.last, o.hits, o.created, o.priority = nid, x["last"], x["hits"], x["created"], x["priority"]
            cands.append((evict_key(t.policy, o), nid))
        if not cands:
            break
        _, nid = min(cands)
        out.append((nid, nodes[nid]["val"]))
        got += len(nodes[nid]["val"])
        del nodes[nid]
    return out


@pytest.mark.parametrize("policy", POLICIES)
@settings(max_examples=60, deadline=None)
@given(seqs=seq_strategy, n=st.integers(1, 30), seed=st.integers(0, 1000), keep=st.integers(0, 3),
       matches=st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=8), max_size=6))
def test_policy_eviction_matches_brute_force(policy, seqs, n, seed, keep, matches):
    rng = random.Random(seed)
    t = OracleTree(200, list(rng.sample(range(200), 200)), policy=policy)
    held = []
    for i, toks in enumerate(seqs):
        bt = driver.prepare_batch(t, [toks])
        t.insert(toks, bt.rows[0], priority=i % 3)
        held.append(bt.last_nodes[0])
    for toks in matches:
        t.match(toks)
    for nid in held[keep:]:
        driver.release(t, [nid])
    expect = brute_evict_policy(t, n)
    t.evict(n)
    assert [(nid, list(s)) for nid, s in t.take_evlog()] == expect
    check_invariants(t)


def _three_leaves(policy):
    # leaves A=[1,1] (created first), B=[2,2], C=[3,3] under the root, all unlocked
    t = OracleTree(16, policy=policy)
    for toks, prio in (([1, 1], 2), ([2, 2], 0), ([3, 3], 1)):
        bt = driver.prepare_batch(t, [toks])
        t.insert(toks, bt.rows[0], priority=prio)
        driver.release(t, bt.last_nodes)
    return t


def evicted_key_first(t):
    t.evict(1)
    log = t.take_evlog()
    return log[0][1]


def test_policy_orders_on_a_hand_example():
    # slots: A -> [0,1], B -> [2,3], C -> [4,5]; then A is matched twice, C once
    def prep(policy):
        t = _three_leaves(policy)
        t.match([1, 1])
        t.match([1, 1])
        t.match([3, 3])
        return t
    assert evicted_key_first(prep("lru")) == [2, 3]        # B: least recently used
    assert evicted_key_first(prep("mru")) == [4, 5]        # C: most recently used
    assert evicted_key_first(prep("fifo")) == [0, 1]       # A: created first
    assert evicted_key_first(prep("filo")) == [4, 5]       # C: created last
    assert evicted_key_first(prep("lfu")) == [2, 3]        # B: never hit
    assert evicted_key_first(prep("priority")) == [2, 3]   # B: priority 0
    t = prep("slru")                                       # A protected (2 hits); B, C probationary
    assert evicted_key_first(t) == [2, 3]
    assert evicted_key_first(t) == [4, 5]
    assert evicted_key_first(t) == [0, 1]


def test_hit_count_and_created_across_a_split():
    t = OracleTree(16)
    bt = driver.prepare_batch(t, [[1, 2, 3, 4]])     # leaf created by this insert
    driver.release(t, bt.last_nodes)
    c0 = [c for _, _, c, _ in t.dump_stats()][0]
    t.match([1, 2, 3, 4])                              # full hit: hits 1
    t.match([1, 2, 9])                                 # partial: split at 2
    stats = {tuple(t.path_tokens(nid)): (h, c) for nid, h, c, _ in t.dump_stats()}
    assert stats[(1, 2)] == (2, c0) and stats[(1, 2, 3, 4)] == (1, c0)


def test_peek_changes_nothing():
    t = OracleTree(32)
    for toks in ([1, 2, 3, 4], [1, 2, 5], [7]):
        driver.release(t, driver.prepare_batch(t, [toks]).last_nodes)
    before = (t.dump(), t.dump_stats(), t.clock)
    assert t.peek([1, 2, 3, 9]) == 3 and t.peek([1, 2]) == 2 and t.peek([8]) == 0 and t.peek([7, 7]) == 1
    assert (t.dump(), t.dump_stats(), t.clock) == before


def test_priority_raised_by_walking_inserts_hand_example():
    """Priority field ([RC] "삽입: _insert_helper" passes a priority down the walk): an insert
    raises every node it walks over to max(old, its priority), a cut raises only the upper part
    (the part holding walked positions), a new node takes the insert's priority.  Expected values
    derived by hand below."""
    t = _three_leaves("priority")          # A=[1,1] prio 2, B=[2,2] prio 0, C=[3,3] prio 1 (ids 1, 2, 3)
    prio = {tuple(t.path_tokens(nid)): p for nid, _, _, p in t.dump_stats()}
    assert prio == {(1, 1): 2, (2, 2): 0, (3, 3): 1}
    # insert [2, 7] at priority 5: B is cut after its first position; upper [2] is walked (5),
    # lower [2] keeps 0, the new node [7] takes 5
    bt = driver.prepare_batch(t, [[2, 7]])
    t.insert([2, 7], bt.rows[0], priority=5)
    driver.release(t, bt.last_nodes)
    prio = {tuple(t.path_tokens(nid)): p for nid, _, _, p in t.dump_stats()}
    assert prio == {(1, 1): 2, (2,): 5, (2, 2): 0, (2, 7): 5, (3, 3): 1}
    # priority order: lowest first, ties by access time: (2,2) prio 0, then C prio 1, then A prio 2;
    # [2] is not a leaf until both children are gone
    got = []
    for _ in range(3):
        t.evict(1)
        got += [list(s) for _, s in t.take_evlog()]
    assert got == [[3], [4, 5], [0, 1]]    # lower half of B (its second slot), C, A
