"""Oracle sequential driver: batches of requests -> slot tables.  TEST INFRASTRUCTURE ONLY.

Per request, in arrival order (radix-cache walkthrough page, sections "프리픽스 매칭",
"삽입", "참조 카운트"; the RadixAttention explainer's matching formula: the matched
length needs no recompute and only the rest is prefilled):
  1. match the full token list -> matched length m, its slots, node a;
  2. lock a (so the allocation below cannot evict the reused prefix);
  3. allocate L - m fresh slots (evicting LRU leaves on shortfall);
  4. insert (tokens, prefix slots ++ fresh slots) -> already-cached length t and
     the node ending the key; t equals m because nothing between 1 and 4 can add
     to the tree and the locked path cannot be evicted;
  5. lock the new end node, unlock a;
  6. the request's slot row is prefix slots ++ fresh slots; it extends positions [m, L).
After the batch's kernels the end nodes are unlocked (release).

Decode (one query token per sequence per step): one allocation of B slots per step,
slot i going to sequence i, appended to its row.  When the sequences finish, each
full token list (prompt + decoded tokens) is inserted with its full row and the
prompt's end node is unlocked (the overview page's feedback loop from generated
tokens back to insertion, applied at request granularity).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from .radix_tree import OracleError, OracleTree


@dataclasses.dataclass
class BatchTables:
    rows: List[List[int]]        # full slot row per request
    prefix_lens: List[int]
    extend_lens: List[int]
    last_nodes: List[int]
    new_slots: List[int]         # fresh slots, concatenated in request order (= extend rows)


def prepare_batch(tree: OracleTree, token_lists: Sequence[Sequence[int]],
                  priorities: Optional[Sequence[int]] = None) -> BatchTables:
    """Steps 1-6 for each request in order; request i's insert carries priorities[i]
    (default 0), the priority argument of the radix-cache page's insert helper."""
    out = BatchTables([], [], [], [], [])
    for i, toks in enumerate(token_lists):
        toks = [int(t) for t in toks]
        m, ps, a = tree.match(toks)
        tree.inc_lock(a)
        try:
            ns = tree.alloc(len(toks) - m)
        except OracleError:
            tree.dec_lock(a)          # a failed request leaves no lock behind
            raise
        t, last = tree.insert(toks, ps + ns, 0 if priorities is None else int(priorities[i]))
        if t != m:
            raise OracleError(f"insert found {t} cached tokens after a match of {m}")
        tree.inc_lock(last)
        tree.dec_lock(a)
        out.rows.append(ps + ns)
        out.prefix_lens.append(m)
        out.extend_lens.append(len(toks) - m)
        out.last_nodes.append(last)
        out.new_slots.extend(ns)
    return out


def release(tree: OracleTree, nodes: Sequence[int]) -> None:
    for n in nodes:
        tree.dec_lock(n)


def decode_alloc(tree: OracleTree, rows: List[List[int]]) -> List[int]:
    """One decode step: one slot per sequence, appended to its row."""
    slots = tree.alloc(len(rows))
    for r, s in zip(rows, slots):
        r.append(s)
    return slots


def finish(tree: OracleTree, token_lists: Sequence[Sequence[int]], rows: Sequence[Sequence[int]],
           prompt_lens: Sequence[int], last_nodes: Sequence[int]) -> List[int]:
    """Insert finished sequences (prompt + decoded tokens) and unlock their prompt end nodes.

    Positions [prompt_len, t) that the insert finds already cached keep the tree's slots;
    the sequence's own slots for them are returned to the free list (the radix-cache
    page: the caller frees the duplicate indices reported by insert)."""
    ends = []
    for toks, row, plen, a in zip(token_lists, rows, prompt_lens, last_nodes):
        t, end = tree.insert(list(toks), list(row))
        if t > plen:
            tree.free_slots(list(row)[plen:t])
        tree.dec_lock(a)
        ends.append(end)
    return ends


@dataclasses.dataclass
class RunLog:
    """Everything the host side of a workload produces, for bit-exact comparison."""
    batches: List[BatchTables]
    decode_slots: List[List[int]]
    evlog: list
    free: List[int]
    evictable: int
    protected: int
    dump: list


def run_workload_host(wl, release_last_batch: bool = True, policy: str = "lru") -> RunLog:
    """Drive a ``workloads.Workload`` through the oracle tree (host side only)."""
    tree = OracleTree(wl.pool_slots, wl.free_order, policy)
    batches = []
    for r in wl.pre_insert:
        bt = prepare_batch(tree, [r.tokens])
        release(tree, bt.last_nodes)
    for bi, batch in enumerate(wl.batches):
        bt = prepare_batch(tree, [r.tokens for r in batch])
        batches.append(bt)
        if bi < len(wl.batches) - 1:
            release(tree, bt.last_nodes)
    dec = []
    steps = int(wl.decode_tokens.shape[0])
    last = batches[-1]
    rows = [list(r) for r in last.rows]
    for s in range(steps):
        dec.append(decode_alloc(tree, rows))
    if steps:
        toks = [list(r.tokens) + wl.decode_tokens[:, i].tolist() for i, r in enumerate(wl.batches[-1])]
        plens = [len(r.tokens) for r in wl.batches[-1]]
        finish(tree, toks, rows, plens, last.last_nodes)
    elif release_last_batch:
        release(tree, last.last_nodes)
    return RunLog(batches, dec, tree.take_evlog(), list(tree.free), tree.evictable,
                  tree.protected, tree.dump())


def req_to_token(rows: Sequence[Sequence[int]], stride: int) -> np.ndarray:
    out = np.full((len(rows), stride), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out
