"""Pins for the oracle's batch driver beyond prepare_batch: the decode-step allocation and the
finish of sequences (insert of prompt + decoded tokens, release of the caller's duplicate slots,
unlock), against hand-derived expected values (tests/golden/finish_duplicates.json, derivation
written out in the file)."""
import json
import os

from oracle import driver
from oracle.radix_tree import OracleTree

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_prepare_decode_finish_hand_example():
    g = load("finish_duplicates.json")
    t = OracleTree(g["pool_slots"])
    bt = driver.prepare_batch(t, g["prompts"])
    assert bt.prefix_lens == g["prefix_lens"] and bt.extend_lens == g["extend_lens"]
    assert bt.new_slots == g["new_slots"] and bt.last_nodes == g["last_nodes"]
    assert bt.rows == g["rows_after_prepare"]
    # every prompt holds its path: 5 cached tokens, all protected
    assert (t.evictable, t.protected) == (0, 5)
    rows = [list(r) for r in bt.rows]
    dec = [driver.decode_alloc(t, rows) for _ in range(len(g["decode_slots"]))]
    assert dec == g["decode_slots"]
    # slot i of each step goes to sequence i, appended to its row
    for i, r in enumerate(rows):
        assert r == g["rows_after_prepare"][i] + [s[i] for s in g["decode_slots"]]
    full = [p + d for p, d in zip(g["prompts"], g["decode_tokens"])]
    ends = driver.finish(t, full, rows, [len(p) for p in g["prompts"]], bt.last_nodes)
    assert ends == g["ends"]
    assert list(t.free) == g["free_after_finish"]
    assert (t.evictable, t.protected, t.clock) == (g["evictable"], g["protected"], g["clock_after_finish"])
    assert [list(x[:4]) + [list(x[4]), list(x[5])] for x in t.dump()] == g["dump_after_finish"]
    # the first finished sequence's decode slots are what a later request reuses
    m, slots, node = t.match(g["followup_query"])
    assert (m, slots, node) == (g["followup_match_len"], g["followup_match_slots"], g["followup_node"])


def test_finish_frees_only_positions_past_the_prompt():
    """A finished sequence whose whole prompt and decode run are already cached gives back exactly
    its decode slots; a prompt position can never be a duplicate (the prompt's own insert cached
    it), and slot conservation holds: free + cached + in flight = capacity."""
    t = OracleTree(32)
    bt = driver.prepare_batch(t, [[5, 6], [5, 6]])
    rows = [list(r) for r in bt.rows]
    for _ in range(3):
        driver.decode_alloc(t, rows)
    full = [[5, 6, 1, 2, 3], [5, 6, 1, 2, 3]]
    driver.finish(t, full, rows, [2, 2], bt.last_nodes)
    assert list(t.free)[-3:] == rows[1][2:]           # the second sequence's three decode slots
    assert len(t.free) + t.cached_tokens() == 32
    assert t.protected == 0 and t.evictable == 5
