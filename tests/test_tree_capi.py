"""The C-ABI library on the CPU: every declared symbol is exported, and the C++ radix tree and
slot allocator agree bit-exactly with the oracle (match lengths, slot rows, node ids, access
stamps, lock counts, eviction log, free list) on the worked example, random operation
streams, error paths and the host side of every workload."""
import json
import os
import random
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import prefix_shared_kv_match_amd as pkv
from prefix_shared_kv_match_amd import runtime
from oracle import driver
from oracle.radix_tree import OracleError, OracleTree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def header_functions():
    src = open(os.path.join(ROOT, "include", "pkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**\s*((?:rt|pkv)_[a-z0-9_]+)\s*\(",
                                 src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 30
    lib = pkv.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(pkv._capi.SIGNATURES), set(names) ^ set(pkv._capi.SIGNATURES)


def test_worked_example_through_capi():
    with open(os.path.join(GOLDEN, "radix_worked_example.json")) as f:
        g = json.load(f)
    t = pkv.rt_create(g["pool_slots"])
    try:
        for toks in g["inserts"]:
            hb = runtime.prepare(t, [np.array(toks)], 16)
            pkv.rt_release(t, hb.last_nodes)
        m, slots, _ = pkv.rt_match_prefix(t, g["query"])
        assert m == g["match_len"] and slots.tolist() == g["match_slots"]
        nodes = {n[4]: n[5] for n in pkv.rt_dump(t)}
        for n in g["tree"]:
            assert list(nodes[tuple(n["key"])]) == n["kv"]
    finally:
        pkv.rt_destroy(t)


class Pair:
    """The oracle tree and the library tree driven with the same operations."""

    def __init__(self, pool_slots, free_order=None):
        self.o = OracleTree(pool_slots, free_order)
        self.t = pkv.rt_create(pool_slots, free_order)

    def close(self):
        pkv.rt_destroy(self.t)

    def same(self):
        assert pkv.rt_dump(self.t) == self.o.dump()
        assert pkv.rt_copy_free_list(self.t).tolist() == list(self.o.free)
        assert pkv.rt_evictable_size(self.t) == self.o.evictable
        assert pkv.rt_protected_size(self.t) == self.o.protected
        assert pkv.rt_clock(self.t) == self.o.clock
        assert pkv.rt_take_eviction_log(self.t) == [(i, list(s)) for i, s in self.o.take_evlog()]


def both(fo, fl):
    """Run an oracle op and the library op; both must succeed or both must fail."""
    try:
        ro = fo()
        eo = None
    except OracleError as e:
        ro, eo = None, e
    try:
        rl = fl()
        el = None
    except pkv.PkvError as e:
        rl, el = None, e
    assert (eo is None) == (el is None), (eo, el)
    return ro, rl


ops = st.lists(st.tuples(st.sampled_from(["prep", "match", "insert_raw", "release", "evict", "alloc", "free",
                                          "decode"]),
                         st.lists(st.integers(0, 3), min_size=0, max_size=9), st.integers(0, 12)),
               min_size=1, max_size=40)


@settings(max_examples=250, deadline=None)
@given(seq=ops, cap=st.integers(6, 40), seed=st.integers(0, 10_000))
def test_random_operation_streams_match_oracle(seq, cap, seed):
    rng = random.Random(seed)
    pool = cap + rng.randrange(0, 5)
    order = rng.sample(range(pool), cap)
    P = Pair(pool, order)
    held = []          # (oracle node, library node)
    inflight = []      # slots handed out by alloc
    try:
        for op, toks, n in seq:
            if op == "prep" and toks:
                ro, rl = both(lambda: driver.prepare_batch(P.o, [toks]),
                              lambda: runtime.prepare(P.t, [np.array(toks)], 16))
                if ro is not None:
                    assert rl.prefix_lens.tolist() == ro.prefix_lens
                    assert rl.req_to_token[0, :len(toks)].tolist() == ro.rows[0]
                    assert rl.new_slots.tolist() == ro.new_slots
                    assert rl.last_nodes.tolist() == ro.last_nodes
                    held.append(ro.last_nodes[0])
            elif op == "match":
                ro, rl = both(lambda: P.o.match(toks), lambda: pkv.rt_match_prefix(P.t, toks))
                assert (ro[0], list(ro[1]), ro[2]) == (rl[0], rl[1].tolist(), rl[2])
            elif op == "insert_raw" and toks and len(inflight) >= len(toks):
                vals = inflight[:len(toks)]
                # the library refuses new-leaf slots that are not in flight; the oracle does not check,
                # so only compare when the uncached part is covered by in-flight slots (always, here)
                ro, rl = both(lambda: P.o.insert(toks, vals), lambda: pkv.rt_insert(P.t, toks, vals))
                assert ro == rl
                m = ro[0]
                del inflight[m:len(toks)]          # now cached
                # the duplicates [0, m) stay in flight
            elif op == "release" and held:
                nid = held.pop(rng.randrange(len(held)))
                both(lambda: P.o.dec_lock(nid), lambda: pkv.rt_dec_lock_ref(P.t, nid))
            elif op == "evict":
                ro, rl = both(lambda: P.o.evict(n), lambda: pkv.rt_evict(P.t, n))
                assert ro == rl
            elif op == "alloc":
                ro, rl = both(lambda: P.o.alloc(n), lambda: pkv.rt_alloc(P.t, n))
                if ro is not None:
                    assert ro == rl.tolist()
                    inflight.extend(ro)
            elif op == "free" and inflight:
                k = min(n, len(inflight))
                s = inflight[:k]
                both(lambda: P.o.free_slots(s), lambda: pkv.rt_free(P.t, s))
                del inflight[:k]
            elif op == "decode" and held:
                # one decode-style allocation for a pseudo batch
                ro, rl = both(lambda: P.o.alloc(2), lambda: pkv.rt_alloc(P.t, 2))
                if ro is not None:
                    inflight.extend(ro)
            P.same()
    finally:
        P.close()


def test_error_paths_match():
    P = Pair(8)
    try:
        hb = runtime.prepare(P.t, [np.array([1, 2, 3, 4, 5, 6])], 8)
        bo = driver.prepare_batch(P.o, [[1, 2, 3, 4, 5, 6]])
        with pytest.raises(pkv.PkvError) as e:
            runtime.prepare(P.t, [np.array([9, 9, 9])], 8)
        assert e.value.code == -2                       # OOM: the locked leaf cannot go
        with pytest.raises(OracleError):
            driver.prepare_batch(P.o, [[9, 9, 9]])
        P.same()
        pkv.rt_release(P.t, hb.last_nodes)
        driver.release(P.o, bo.last_nodes)
        with pytest.raises(pkv.PkvError) as e:
            pkv.rt_release(P.t, hb.last_nodes)
        assert e.value.code == -3                       # unlock below zero
        with pytest.raises(pkv.PkvError) as e:
            pkv.rt_free(P.t, [7])                       # slot 7 is free, not in flight
        assert e.value.code == -4
        with pytest.raises(pkv.PkvError) as e:
            pkv.rt_inc_lock_ref(P.t, 999)
        assert e.value.code == -5
        got = pkv.rt_alloc(P.t, 4)                      # evicts the 6-token leaf
        assert got.tolist() == P.o.alloc(4)
        with pytest.raises(pkv.PkvError) as e:
            pkv.rt_inc_lock_ref(P.t, int(hb.last_nodes[0]))   # stale id after eviction
        assert e.value.code == -5
        with pytest.raises(pkv.PkvError):
            pkv.rt_insert(P.t, [5, 5], [got[0], got[0]])       # repeated slot
        with pytest.raises(pkv.PkvError):
            pkv.rt_insert(P.t, [5, 5], [4, 5])                 # free slots, not in flight
        P.same()
    finally:
        P.close()
    with pytest.raises(pkv.PkvError):
        pkv.rt_create(4, [0, 0, 1])
    with pytest.raises(pkv.PkvError):
        pkv.rt_create(0)


def test_prepare_rejects_small_stride():
    t = pkv.rt_create(64)
    try:
        with pytest.raises(pkv.PkvError):
            runtime.prepare(t, [np.arange(10)], 8)
        assert pkv.rt_free_size(t) == 64 and pkv.rt_dump(t) == []
    finally:
        pkv.rt_destroy(t)


def test_eviction_log_switch():
    """The log records evictions while on (the default), drops its contents when turned off,
    records nothing while off, and the tree itself evicts the same either way."""
    t = pkv.rt_create(16)
    try:
        for key in ([1, 2, 3], [4, 5], [6]):
            pkv.rt_release(t, runtime.prepare(t, [np.array(key)], 8).last_nodes)
        assert pkv.rt_evict(t, 3) == 3                  # [1, 2, 3] (oldest) goes first
        pkv.rt_set_eviction_log(t, False)
        assert pkv.rt_take_eviction_log(t) == []        # turning it off dropped the entry
        assert pkv.rt_evict(t, 2) == 2
        assert pkv.rt_take_eviction_log(t) == []
        pkv.rt_set_eviction_log(t, True)
        assert pkv.rt_evict(t, 1) == 1
        log = pkv.rt_take_eviction_log(t)
        assert len(log) == 1 and len(log[0][1]) == 1
        assert pkv.rt_free_size(t) == 16 and pkv.rt_dump(t) == []
    finally:
        pkv.rt_destroy(t)


def test_runtime_prepare_into_given_rows():
    """prepare() writes the slot rows into a caller's array (the staged upload path) and
    leaves entries past each request's length untouched."""
    t = pkv.rt_create(64)
    try:
        rows = np.full((2, 8), 77, dtype=np.int32)
        hb = runtime.prepare(t, [np.array([1, 2, 3]), np.array([1, 2, 9, 9])], 8, r2t=rows)
        assert hb.req_to_token.base is rows or hb.req_to_token is rows or np.shares_memory(hb.req_to_token, rows)
        assert rows[0, :3].tolist() == [0, 1, 2] and rows[1, :4].tolist() == [0, 1, 3, 4]
        assert rows[0, 3:].tolist() == [77] * 5 and rows[1, 4:].tolist() == [77] * 4
    finally:
        pkv.rt_destroy(t)


def compare_workload(wl):
    ob = driver.run_workload_host(wl)
    lb, ldec, levlog, lfree, lev, lprot, ldump = runtime.run_workload_host(wl)
    assert len(ob.batches) == len(lb)
    for o, l in zip(ob.batches, lb):
        assert l.prefix_lens.tolist() == o.prefix_lens
        assert l.extend_lens.tolist() == o.extend_lens
        assert l.last_nodes.tolist() == o.last_nodes
        assert l.new_slots.tolist() == o.new_slots
        for i, row in enumerate(o.rows):
            assert l.req_to_token[i, :len(row)].tolist() == row
    assert ldec == ob.decode_slots
    assert levlog == [(i, list(s)) for i, s in ob.evlog]
    assert lfree == ob.free
    assert (lev, lprot) == (ob.evictable, ob.protected)
    assert ldump == ob.dump
    return ob


def test_workload_tiny_f32_host():
    import workloads
    ob = compare_workload(workloads.tiny_f32())
    assert ob.batches[0].prefix_lens == [0, 64, 64, 64]
    assert ob.batches[0].extend_lens == [80, 16, 16, 16]


def test_workload_fewshot_host():
    import workloads
    ob = compare_workload(workloads.fewshot_bf16())
    assert ob.batches[0].prefix_lens == [1800] * 64


def test_workload_multiturn_host_evicts():
    import workloads
    ob = compare_workload(workloads.multiturn_bf16())
    assert len(ob.evlog) > 0
    hits = sum(sum(b.prefix_lens) for b in ob.batches)
    assert hits > 0


def test_workload_decode_host():
    import workloads
    wl = workloads.decode_bf16(n_seq=96, steps=4)
    ob = compare_workload(wl)
    assert ob.batches[0].prefix_lens == [1024] * 96


def test_workload_longctx_host():
    import workloads
    ob = compare_workload(workloads.longctx_fp8(steps=8))
    assert ob.batches[0].prefix_lens == [32768] * 16


def test_workload_tot_host():
    import workloads
    ob = compare_workload(workloads.tot_bf16())
    # level 1 reuses the root; later levels reuse the root and the parent's path
    assert ob.batches[0].prefix_lens[0] == 1024
    assert all(p >= 1024 for b in ob.batches for p in b.prefix_lens)
    # the template run is shared by siblings: all but the first sibling reuse it
    fam = ob.batches[3]
    for f in range(0, 256, 4):
        assert all(fam.prefix_lens[f + c] == fam.prefix_lens[f] + 8 for c in range(1, 4))


def test_finish_duplicate_release_through_capi():
    """rt_finish's duplicate branch (the caller's slots of positions the final insert finds
    cached go back to the free list): the hand-derived example of
    tests/golden/finish_duplicates.json, bit-exact through the C ABI (tables, decode slots,
    end nodes, free list, counters, clock, every node) and against the oracle."""
    with open(os.path.join(GOLDEN, "finish_duplicates.json")) as f:
        g = json.load(f)
    t = pkv.rt_create(g["pool_slots"])
    o = OracleTree(g["pool_slots"])
    try:
        stride = 8
        hb = runtime.prepare(t, [np.array(p) for p in g["prompts"]], stride)
        ob = driver.prepare_batch(o, g["prompts"])
        assert hb.prefix_lens.tolist() == g["prefix_lens"] == ob.prefix_lens
        assert hb.extend_lens.tolist() == g["extend_lens"]
        assert hb.new_slots.tolist() == g["new_slots"]
        assert hb.last_nodes.tolist() == g["last_nodes"]
        rows = [list(r) for r in ob.rows]
        for s, want in enumerate(g["decode_slots"]):
            out = np.empty(hb.n, dtype=np.int32)
            pkv.rt_decode_step(t, hb.req_to_token, hb.seq_lens, out)
            assert out.tolist() == want == driver.decode_alloc(o, rows), s
        full = [np.array(p + d) for p, d in zip(g["prompts"], g["decode_tokens"])]
        toks, indptr = runtime.flatten(full)
        ends = pkv.rt_finish(t, toks, indptr, hb.req_to_token, [len(p) for p in g["prompts"]], hb.last_nodes)
        oends = driver.finish(o, [f.tolist() for f in full], rows, [len(p) for p in g["prompts"]], ob.last_nodes)
        assert ends.tolist() == g["ends"] == oends
        assert pkv.rt_copy_free_list(t).tolist() == g["free_after_finish"] == list(o.free)
        assert pkv.rt_evictable_size(t) == g["evictable"] and pkv.rt_protected_size(t) == g["protected"]
        assert pkv.rt_clock(t) == g["clock_after_finish"]
        assert [list(x[:4]) + [list(x[4]), list(x[5])] for x in pkv.rt_dump(t)] == g["dump_after_finish"]
        assert pkv.rt_dump(t) == o.dump()
        m, slots, node = pkv.rt_match_prefix(t, g["followup_query"])
        assert (m, slots.tolist(), node) == (g["followup_match_len"], g["followup_match_slots"], g["followup_node"])
    finally:
        pkv.rt_destroy(t)


@settings(max_examples=60, deadline=None)
@given(prompts=st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=5), min_size=1, max_size=5),
       dec=st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=5), min_size=1, max_size=4))
def test_finish_with_duplicates_matches_oracle(prompts, dec):
    """Random batches over a 3-token vocabulary whose decoded tokens often repeat another
    sequence's: rt_finish bit-exact against the oracle's finish (free list, dump, counters)."""
    steps = len(dec[0])
    dtoks = [(dec[i % len(dec)] * steps)[:steps] for i in range(len(prompts))]
    t = pkv.rt_create(64)
    o = OracleTree(64)
    try:
        hb = runtime.prepare(t, [np.array(p) for p in prompts], 16)
        ob = driver.prepare_batch(o, prompts)
        rows = [list(r) for r in ob.rows]
        for _ in range(steps):
            out = np.empty(hb.n, dtype=np.int32)
            pkv.rt_decode_step(t, hb.req_to_token, hb.seq_lens, out)
            assert out.tolist() == driver.decode_alloc(o, rows)
        full = [p + d for p, d in zip(prompts, dtoks)]
        toks, indptr = runtime.flatten([np.array(f) for f in full])
        ends = pkv.rt_finish(t, toks, indptr, hb.req_to_token, [len(p) for p in prompts], hb.last_nodes)
        assert ends.tolist() == driver.finish(o, full, rows, [len(p) for p in prompts], ob.last_nodes)
        assert pkv.rt_dump(t) == o.dump()
        assert pkv.rt_copy_free_list(t).tolist() == list(o.free)
        assert (pkv.rt_evictable_size(t), pkv.rt_protected_size(t)) == (o.evictable, o.protected)
        assert pkv.rt_free_size(t) + o.cached_tokens() == 64
    finally:
        pkv.rt_destroy(t)
