"""The shared-prefix decode plan (pkv_decode_shared_plan) on the CPU, against brute force over
pairs of slot rows: members is a permutation, every item's members hold its chunk whole and
slot for slot equal, each sequence's chunks 0 .. skip-1 are covered exactly once, and the
plan is maximal (two sequences that agree on chunks 0..k, whole in both contexts, both share
chunk k).  On rows built the way the radix tree builds them, the last-slot shortcut
(rows_from_tree) gives the same plan.  With private_items the same shared items come first and
one-member items then cover every sequence's remaining chunks, once each."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import prefix_shared_kv_match_amd as pkv


def rows_from_paths(rng, paths, lens, chunk, stride):
    """Slot rows of sequences that follow paths in a tree of chunks: equal path prefixes give
    equal slots (as the radix tree hands them out), the rest is private."""
    r2t = np.full((len(paths), stride), -1, dtype=np.int32)
    node_slots = {}
    nxt = 0
    for b, (path, L) in enumerate(zip(paths, lens)):
        for k in range((L + chunk - 1) // chunk):
            key = tuple(path[:k + 1]) if k < len(path) else ("private", b, k)
            if key not in node_slots:
                node_slots[key] = np.arange(nxt, nxt + chunk, dtype=np.int32)
                nxt += chunk
            hi = min(L, (k + 1) * chunk)
            r2t[b, k * chunk:hi] = node_slots[key][:hi - k * chunk]
    perm = rng.permutation(nxt).astype(np.int32)        # slots are not in any particular order
    return np.where(r2t >= 0, perm[np.maximum(r2t, 0)], -1).astype(np.int32)


def check_plan(r2t, lens, chunk, rows, members, skip, items, max_span=1):
    b = len(lens)
    assert items.shape[1:] == (4,)
    assert sorted(members.tolist()) == list(range(b))
    full = [L // chunk for L in lens]
    covered = {i: [] for i in range(b)}
    job_sizes = {}
    for m0, nm, k0, span in items.tolist():
        assert 1 <= nm <= rows and 0 <= m0 and m0 + nm <= b and 1 <= span <= max_span
        mem = members[m0:m0 + nm].tolist()
        for k in range(k0, k0 + span):
            for i in mem:
                assert full[i] > k
                covered[i].append(k)
            for i in mem[1:]:
                assert np.array_equal(r2t[i, :(k + 1) * chunk], r2t[mem[0], :(k + 1) * chunk])
            key = (k, tuple(r2t[mem[0], :(k + 1) * chunk]))
            job_sizes[key] = job_sizes.get(key, 0) + nm
    for i in range(b):
        assert sorted(covered[i]) == list(range(skip[i])), (i, covered[i], skip[i])
    # every chunk listed for a sequence is shared with another one: jobs have >= 2 members
    assert all(v >= 2 for v in job_sizes.values())
    # maximal: agreement on chunks 0..k (whole in both) means both cover chunk k
    for i in range(b):
        for j in range(i + 1, b):
            k = 0
            while k < min(full[i], full[j]) and np.array_equal(r2t[i, k * chunk:(k + 1) * chunk],
                                                               r2t[j, k * chunk:(k + 1) * chunk]):
                k += 1
            assert skip[i] >= k and skip[j] >= k, (i, j, k, skip[i], skip[j])


def check_private(r2t, lens, chunk, rows, max_span, rows_from_tree=False):
    """The private-items plan: the shared plan's members and items first, then one-member items
    of at most max_span chunks covering chunks skip[b] .. ceil(L / chunk) - 1 of each sequence
    exactly once; skip[b] = ceil(L / chunk)."""
    m0, s0, i0 = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree, max_span)
    m, s, it = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree, max_span, private_items=True)
    n0 = len(i0)
    assert np.array_equal(m, m0) and np.array_equal(it[:n0], i0)
    ends = [(L + chunk - 1) // chunk for L in lens]
    assert s.tolist() == ends
    covered = {b: [] for b in range(len(lens))}
    for m_0, nm, k0, span in it[n0:].tolist():
        assert nm == 1 and 1 <= span <= max_span and 0 <= m_0 < len(lens)
        covered[int(m[m_0])] += list(range(k0, k0 + span))
    for b in range(len(lens)):
        assert sorted(covered[b]) == list(range(s0[b], ends[b])), (b, covered[b], s0[b], ends[b])


def test_fewshot_like_one_group():
    rng = np.random.default_rng(0)
    chunk, stride = 64, 640
    lens = [int(x) for x in rng.integers(450, 640, size=20)]
    paths = [[0, 1, 2, 3, 4, 5] for _ in lens]            # a 384-token common prefix (6 chunks)
    r2t = rows_from_paths(rng, paths, lens, chunk, stride)
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 8)
    check_plan(r2t, lens, chunk, 8, members, skip, items)
    assert skip.tolist() == [6] * 20
    assert len(items) == 6 * 3                            # 20 members in items of <= 8
    assert items[:3, 2].tolist() == [0, 0, 0] and items[:3, 1].tolist() == [8, 8, 4]
    assert items[:, 3].tolist() == [1] * 18
    # spans of up to 4 chunks: chunks 0-3 and 4-5, three items each
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 8, max_span=4)
    check_plan(r2t, lens, chunk, 8, members, skip, items, max_span=4)
    assert items[:, 2:].tolist() == [[0, 4]] * 3 + [[4, 2]] * 3
    # private items: every sequence's chunks from 6 to the one holding its newest token
    check_private(r2t, lens, chunk, 8, 4)
    # shared: 3 spans of 2 chunks x 3 items, then the private ones
    m, s, it = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 8, max_span=2, private_items=True)
    assert all(nm == 1 for nm in it[9:, 1]) and len(it) == 9 + sum(((L + 63) // 64 - 6 + 1) // 2 for L in lens)


def test_tree_shaped_sharing_and_singletons():
    rng = np.random.default_rng(1)
    chunk, stride = 64, 512
    paths = [[0, 1, 2], [0, 1, 3], [0, 4], [0, 4], [5], [0, 1, 2], [6, 7]]
    lens = [300, 300, 250, 130, 200, 190, 500]
    r2t = rows_from_paths(rng, paths, lens, chunk, stride)
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 16)
    check_plan(r2t, lens, chunk, 16, members, skip, items)
    # 0 and 5 share 3 chunks but 5 holds only 2 whole (190 tokens); 0, 1 share 2; 2, 3 share 2
    # (3 holds 2 whole); chunk 0 is shared by 0, 1, 2, 3, 5
    assert skip.tolist() == [2, 2, 2, 2, 0, 2, 0]


def test_no_sharing_and_short_contexts():
    rng = np.random.default_rng(2)
    lens = [1, 63, 64, 65, 200]
    r2t = rows_from_paths(rng, [[i] for i in range(5)], lens, 64, 256)
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, 64, 32)
    assert len(items) == 0 and skip.tolist() == [0] * 5
    members, skip, items = pkv.pkv_decode_shared_plan(r2t[:0], [], 64, 32)
    assert len(items) == 0 and members.size == 0


def test_same_first_slot_different_chunk_does_not_share():
    """Rows that agree on a chunk's first slot but not on the rest of it (not something the tree
    produces) are not grouped."""
    r2t = np.arange(4 * 128, dtype=np.int32).reshape(4, 128)
    r2t[1] = r2t[0]
    r2t[1, 5] = 999
    r2t[2] = r2t[0]
    lens = [128, 128, 128, 100]
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, 64, 32)
    check_plan(r2t, lens, 64, 32, members, skip, items)
    assert skip.tolist() == [2, 0, 2, 0]


def test_rejects_bad_arguments():
    r2t = np.zeros((2, 128), dtype=np.int32)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_shared_plan(r2t, [10, 10], 100, 8)      # chunk not a multiple of 64
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_shared_plan(r2t, [10, 129], 64, 8)      # longer than the row
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_shared_plan(r2t, [0, 10], 64, 8)        # empty sequence
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_shared_plan(r2t, [10, 10], 64, 8, max_span=0)


@settings(max_examples=150, deadline=None)
@given(seed=st.integers(0, 10_000), n=st.integers(1, 24), depth=st.integers(1, 6), branch=st.integers(1, 3),
       rows=st.sampled_from([1, 2, 16, 128]), max_span=st.sampled_from([1, 2, 3, 8]))
def test_random_trees_against_brute_force(seed, n, depth, branch, rows, max_span):
    rng = np.random.default_rng(seed)
    chunk, stride = 64, 64 * 8
    paths = [[int(x) for x in rng.integers(0, branch, size=depth)] for _ in range(n)]
    lens = [int(x) for x in rng.integers(1, stride + 1, size=n)]
    r2t = rows_from_paths(rng, paths, lens, chunk, stride)
    members, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, max_span=max_span)
    check_plan(r2t, lens, chunk, rows, members, skip, items, max_span)
    # rows built like the tree builds them: the last-slot shortcut gives the same plan
    m2, s2, i2 = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree=True, max_span=max_span)
    assert np.array_equal(m2, members) and np.array_equal(s2, skip) and np.array_equal(i2, items)
    check_private(r2t, lens, chunk, rows, max_span, rows_from_tree=seed % 2 == 0)


def test_first_split_at_current_lengths():
    """The split phase's first chunk for a plan kept while the sequences grow: none while the
    items cover every context, then the skip of the first sequence that grows past them."""
    from prefix_shared_kv_match_amd.runtime import Engine
    rng = np.random.default_rng(3)
    chunk, stride = 64, 512
    paths = [[0, 1, 2], [0, 1, 2], [0, 1, 3], [4]]
    lens = np.array([200, 256, 190, 100])
    r2t = rows_from_paths(rng, paths, lens.tolist(), chunk, stride)
    m, skip, it = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 16, private_items=True)
    assert skip.tolist() == [4, 4, 3, 2]
    assert Engine.first_split(skip, lens, chunk) == Engine.NO_SPLIT_PHASE
    assert Engine.first_split(skip, lens + 1, chunk) == 4          # sequence 1 reaches chunk 4
    assert Engine.first_split(skip, lens + 3, chunk) == 3          # sequence 2 reaches chunk 3
    _, s0, _ = pkv.pkv_decode_shared_plan(r2t, lens, chunk, 16)   # shared chunks only
    assert s0.tolist() == [3, 3, 2, 0] and Engine.first_split(s0, lens, chunk) == 0


@settings(max_examples=80, deadline=None)
@given(seed=st.integers(0, 10_000), n=st.integers(1, 40), hkv=st.sampled_from([1, 4, 8, 32]),
       resident=st.sampled_from([1, 16, 512]), private_max=st.sampled_from([0, 64, 4096, 1 << 20]))
def test_plan_choices_of_the_library(seed, n, hkv, resident, private_max):
    """pkv_decode_plan (the library's choices) equals pkv_decode_shared_plan called the way its
    documentation states: private items when items plus private tails need at most
    private_max_workgroups workgroups (times hkv); the span in 1 .. min(longest context in
    chunks, 64) with the lowest ceil(items x hkv / resident) x (4 + span x chunk / 64), the
    longer one on a tie; and first_split at these lengths."""
    rng = np.random.default_rng(seed)
    chunk, stride, rows = 64, 512, 8
    paths = [[int(x) for x in rng.integers(0, 3, size=4)] for _ in range(n)]
    lens = [int(x) for x in rng.integers(1, stride + 1, size=n)]
    r2t = rows_from_paths(rng, paths, lens, chunk, stride)
    got = pkv.pkv_decode_plan(r2t, lens, chunk, rows, hkv, resident, private_max)
    m, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree=True)
    if items.shape[0] == 0:
        assert got is None
        return
    tails = int(sum((L + chunk - 1) // chunk for L in lens) - skip.sum())
    priv = (items.shape[0] + tails) * hkv <= private_max
    longest = max((L + chunk - 1) // chunk for L in lens)
    costs = {}
    for span in range(1, min(longest, 64) + 1):
        k = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree=True, max_span=span,
                                       private_items=priv)[2].shape[0]
        costs[span] = -(-k * hkv // resident) * (4 + span * chunk // 64)
    best = max(s for s, c in costs.items() if c == min(costs.values()))
    m, skip, items = pkv.pkv_decode_shared_plan(r2t, lens, chunk, rows, rows_from_tree=True, max_span=best,
                                                private_items=priv)
    gm, gs, gi, first = got
    assert np.array_equal(gm, m) and np.array_equal(gs, skip) and np.array_equal(gi, items)
    assert first == pkv.pkv_decode_first_split(skip, lens, chunk)
    need = [s for s, L in zip(skip.tolist(), lens) if (L + chunk - 1) // chunk > s]
    assert first == (min(need) if need else pkv.PKV_NO_SPLIT_PHASE)


def test_plan_span_fills_one_round_on_the_long_context_shape():
    """The span choice on the long-context decode shape (16 sequences over one 32,768-token
    prefix with 1,088-token private tails, chunk 256, 8 kv heads, private items): span 3 would
    make 600 workgroups, two rounds of 512; span 4 makes exactly 512, one round, and is taken."""
    rng = np.random.default_rng(5)
    n, chunk, pre, tail = 16, 256, 32768, 1088
    stride = pre + tail
    shared = rng.permutation(1 << 20)[: pre + n * tail].astype(np.int32)
    r2t = np.zeros((n, stride), dtype=np.int32)
    for i in range(n):
        r2t[i, :pre] = shared[:pre]
        r2t[i, pre:] = shared[pre + i * tail: pre + (i + 1) * tail]
    lens = [stride] * n
    members, skip, items, first = pkv.pkv_decode_plan(r2t, lens, chunk, 16, 8, 512, 4096)
    assert first == pkv.PKV_NO_SPLIT_PHASE
    assert items.shape[0] * 8 == 512
    assert int(items[:, 3].max()) == 4


def test_first_split_and_plan_reject_bad_arguments():
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_first_split([0, 1], [10, 0], 64)        # a sequence of length 0
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_first_split([0], [10], 0)               # no chunk
    r2t = np.zeros((2, 128), dtype=np.int32)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_plan(r2t, [64, 64], 64, 8, 0, 512, 4096)    # hkv 0
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_plan(r2t, [64, 64], 64, 8, 8, 0, 4096)      # no workgroup target
