"""Oracle serve loop: cache-aware batch scheduling and chunked prefill.  TEST INFRASTRUCTURE ONLY.

Cache-aware scheduling (the RadixAttention explainer and the SGLang overview page: waiting
requests are ordered by the length of their cached prefix, longest first, rather than first
come first served, so that requests sharing a cached prefix run while it is still resident).
Where the pages leave the queue model open this module takes these readings:

- requests arrive in a fixed order; request i may name an earlier request ``after[i]`` (a
  conversation's previous turn) and is eligible only once that request was scheduled in an
  earlier batch;
- the scheduler sees the ``window`` oldest requests not yet scheduled (a bounded waiting
  queue), keeps them in arrival order and picks the first ``batch`` eligible ones of
  * ``fcfs``: arrival order, or
  * ``lpm``: descending cached-prefix length from a read-only walk (peek), ties in arrival
    order;
- the picked batch is prepared with ``driver.prepare_batch`` (match, lock, allocate,
  insert) and released after its kernels; the next batch is then scheduled against the
  updated tree.

The oldest waiting request is always eligible (its predecessor arrived earlier and is no
longer waiting), so every round schedules at least one request.

Chunked prefill (the SGLang runtime-flags page: a cap on the tokens one prefill launch
processes).  Reading: one launch holds at most ``budget`` new (uncached) tokens.  Requests
are taken in order; the head request contributes min(its remaining uncached tokens, the
budget left) tokens, and a request cut by the budget goes on in the next launch.  A chunk
of request r ending at position e is prepared as the truncated token list r[:e]: its
match reuses the earlier chunks (inserted by their own prepare and still locked), so it
extends exactly the positions the chunk adds.  The lock a chunk's prepare takes on its
end node is held until the request's next chunk is prepared (or, for the last chunk,
until the launch is released).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

from .driver import BatchTables, prepare_batch, release
from .radix_tree import OracleError, OracleTree

ORDERS = ("fcfs", "lpm")


@dataclasses.dataclass
class ServeLog:
    picks: List[List[int]]           # request indices of each batch, in batch order
    tables: List[BatchTables]
    prompt_tokens: int               # sum of request lengths
    cached_tokens: int               # sum of matched prefix lengths

    @property
    def hit_rate(self) -> float:
        return self.cached_tokens / max(self.prompt_tokens, 1)


def schedule_order(tree: OracleTree, token_lists: Sequence[Sequence[int]], order: str) -> List[int]:
    """Indices of ``token_lists`` in the order the scheduler would take them."""
    idx = list(range(len(token_lists)))
    if order == "fcfs":
        return idx
    if order == "lpm":
        m = [tree.peek(t) for t in token_lists]
        return sorted(idx, key=lambda i: -m[i])       # sorted() is stable: ties stay in arrival order
    raise OracleError(f"unknown scheduling order {order!r}")


def serve(tree: OracleTree, token_lists: Sequence[Sequence[int]], after: Sequence[int], order: str,
          batch: int, window: int, priorities: Optional[Sequence[int]] = None) -> ServeLog:
    if batch < 1 or window < 1:
        raise OracleError("batch and window must be positive")
    n = len(token_lists)
    scheduled = [False] * n
    nxt = 0
    queue: List[int] = []
    log = ServeLog([], [], 0, 0)
    while nxt < n or queue:
        while nxt < n and len(queue) < window:
            queue.append(nxt)
            nxt += 1
        elig = [i for i in queue if after[i] < 0 or scheduled[after[i]]]
        if not elig:
            raise OracleError("no eligible request (a dependency points forward)")
        ordr = schedule_order(tree, [token_lists[i] for i in elig], order)
        pick = [elig[j] for j in ordr[:batch]]
        bt = prepare_batch(tree, [token_lists[i] for i in pick],
                           None if priorities is None else [priorities[i] for i in pick])
        release(tree, bt.last_nodes)
        for i in pick:
            scheduled[i] = True
        queue = [i for i in queue if not scheduled[i]]
        log.picks.append(pick)
        log.tables.append(bt)
        log.prompt_tokens += sum(len(token_lists[i]) for i in pick)
        log.cached_tokens += sum(bt.prefix_lens)
    return log


@dataclasses.dataclass
class ChunkLaunch:
    reqs: List[int]                  # request index of each row group
    ends: List[int]                  # chunk end position of each
    tables: BatchTables              # prepare of the truncated token lists


def chunked_prefill(tree: OracleTree, token_lists: Sequence[Sequence[int]], budget: int) -> List[ChunkLaunch]:
    """Prefill ``token_lists`` (one batch, in order) in launches of at most ``budget`` new tokens."""
    if budget < 1:
        raise OracleError("chunk budget must be positive")
    n = len(token_lists)
    done = [0] * n                   # prefilled length so far (cached prefix included)
    held = [-1] * n                  # end node of the request's last chunk, still locked
    launches: List[ChunkLaunch] = []
    head = 0
    while head < n:
        left = budget
        reqs, ends = [], []
        r = head
        while r < n and left > 0:
            L = len(token_lists[r])
            start = done[r] if held[r] >= 0 else tree.peek(token_lists[r])
            take = min(L - start, left)
            reqs.append(r)
            ends.append(start + take)
            left -= take
            r += 1
        bt = prepare_batch(tree, [list(token_lists[i])[:e] for i, e in zip(reqs, ends)])
        for i, e, last in zip(reqs, ends, bt.last_nodes):
            if held[i] >= 0:
                tree.dec_lock(held[i])
            held[i] = last
            done[i] = e
        launches.append(ChunkLaunch(reqs, ends, bt))
        # requests that reached their end leave the pending range; their lock goes at release
        finished = [i for i in reqs if done[i] >= len(token_lists[i])]
        release(tree, [held[i] for i in finished])
        for i in finished:
            held[i] = -1
        while head < n and done[head] >= len(token_lists[head]) and held[head] < 0:
            head += 1
    return launches
