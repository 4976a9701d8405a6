"""Sanity of the seeded input generators (shapes, determinism, the sibling rule)."""
import numpy as np
import pytest

import workloads


def test_deterministic_and_shapes():
    a = workloads.tiny_f32()
    b = workloads.tiny_f32()
    for ra, rb in zip(a.all_requests, b.all_requests):
        np.testing.assert_array_equal(ra.tokens, rb.tokens)
    np.testing.assert_array_equal(a.free_order, b.free_order)
    np.testing.assert_array_equal(a.values.k([0, 5, 79]), b.values.k([0, 5, 79]))
    assert a.values.k([3]).shape == (1, 8, 64) and a.values.q([3]).shape == (1, 8, 64)
    assert sorted(a.free_order.tolist()) == list(range(1024))
    assert [len(r.tokens) for r in a.batches[0]] == [80] * 4


def test_full_equals_rowwise():
    wl = workloads.fewshot_bf16(n_req=3, prefix_len=700, suffix_range=(5, 9))
    full = wl.values.full(workloads.TAG_K, threads=4)
    rows = np.array([0, 511, 512, 700, wl.values.n_rows - 1])
    np.testing.assert_array_equal(full[rows], wl.values.k(rows))
    # bf16 rounding: low 16 bits are zero
    assert np.all((full.view(np.uint32) & 0xFFFF) == 0)


def equal_token_paths_have_equal_rows(reqs):
    # a trie of token -> (row, children): every equal token path must reach the same row
    trie = {}
    for r in reqs:
        node = trie
        for t, row in zip(r.tokens.tolist(), r.rows.tolist()):
            if t in node:
                assert node[t][0] == row
            else:
                node[t] = (row, {})
            node = node[t][1]


@pytest.mark.parametrize("name", ["tiny_f32", "fewshot_bf16", "multiturn_bf16", "tot_bf16"])
def test_equal_token_paths_carry_equal_rows(name):
    kw = {"n_conv": 40} if name == "multiturn_bf16" else {}
    wl = workloads.make(name, **kw)
    equal_token_paths_have_equal_rows(wl.all_requests)


def test_multiturn_structure():
    wl = workloads.multiturn_bf16()
    reqs = [r for b in wl.batches for r in b]
    assert len(reqs) == 1024 and len(wl.batches) == 32
    assert sum("/branch" in r.tag for r in reqs) == 51
    assert max(len(r.tokens) for r in reqs) <= 8 * 512
    assert len(wl.free_order) == 262_144


def test_fp8_scales():
    wl = workloads.longctx_fp8(prefix_len=600, suffix_len=40, n_req=3, steps=2, pool_slots=2048)
    assert wl.k_scale.shape == (8,) and np.all(wl.k_scale > 0)
    assert np.all(wl.k_inv_scale == (np.float32(1) / wl.k_scale).astype(np.float32))


def test_tot_structure():
    wl = workloads.tot_bf16()
    assert [len(b) for b in wl.batches] == [4, 16, 64, 256]
    assert wl.shape.hq == wl.shape.hkv == 32 and wl.shape.d == 128
    root = wl.pre_insert[0].tokens
    assert len(root) == 1024
    for lvl, batch in enumerate(wl.batches, 1):
        for r in batch:
            assert np.array_equal(r.tokens[:1024], root)
            assert r.tag.count(".") == lvl
    # siblings share the parent's path plus the 8-token template, then differ at the next token
    parent, a, b = wl.batches[0][0], wl.batches[1][0], wl.batches[1][1]
    m = min(len(a.tokens), len(b.tokens))
    assert int(np.argmax(a.tokens[:m] != b.tokens[:m])) == len(parent.tokens) + 8
    # each level's request extends its parent's request
    for parent_i, parent in enumerate(wl.batches[2]):
        for c in range(4):
            child = wl.batches[3][4 * parent_i + c]
            assert np.array_equal(child.tokens[:len(parent.tokens)], parent.tokens)
