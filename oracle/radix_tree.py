"""Oracle radix tree over token ids with a token-granular slot pool.  TEST INFRASTRUCTURE ONLY.

Follows the radix-cache walkthrough page ("[SGLang] RadixAttention: Radix Tree 기반
프리픽스 캐싱의 핵심"):
- a node holds a run of token ids (its key) and one KV slot per token (its value);
  children are keyed by the first token of their key (section "핵심 자료구조: TreeNode");
- the root is never evicted (its lock reference is 1, figure "Radix Tree 구조도");
- match walks down whole children and, on a partial hit, splits the child at the
  match length and stops (section "프리픽스 매칭: match_prefix");
- a split gives the new upper node the first part of the key and value and the
  child's lock reference; the old node keeps the rest (section "노드 분할");
- insert walks like match, counts the already-cached length, and hangs the
  remainder as a new leaf (section "삽입: _insert_helper");
- locking a node counts up every node to the root, moving tokens from the
  evictable to the protected count on 0 -> 1 (section "참조 카운트: lock_ref");
- eviction pops unlocked leaves from a heap, frees their slots, removes them,
  and pushes a parent that becomes an unlocked leaf (section "Eviction 전략").

Readings where the page leaves a step open (each is listed in the design notes):
- access time is a logical clock, +1 per match or insert call; every node visited
  in that call, both halves of a split and any new leaf get the call's value;
- insert splits a partially matched node exactly like match does (the page elides
  that branch) and stamps the nodes it visits;
- the eviction heap key is (access time, node id), ascending; node ids come from a
  creation counter (the split's upper node takes a new id, the lower keeps its id);
- eviction removes whole leaves and stops once at least the requested number of
  tokens is freed;
- the free list is first-in first-out: allocation pops from the head, frees append
  to the tail in the order given;
- allocation evicts (requested - free) tokens when the free list is short, then
  fails with OOM if it is still short.

Eviction policies (the page names lru, lfu, slru, fifo, mru, filo and priority as
strategy objects without their keys; these are the readings taken, each an ascending
heap key ending in the node id so the order is total):
- lru (default): (last access, id)            - mru: (-last access, id)
- fifo: (created, id)                          - filo: (-created, id)
- lfu: (hit count, last access, id)            - priority: (priority, last access, id)
- slru: (protected, last access, id), protected = hit count >= 2 (probationary first)
Node fields behind them: hit count = number of match calls that reused at least one of the
node's tokens (a split's upper half takes the old count + 1, the lower half keeps the old
count); created = clock of the insert that first cached the node's first token (a split's
upper half inherits it); priority = max of the priorities of the inserts through the node
(a split's upper half inherits it, as the page's split code copies priority).
"""
from __future__ import annotations

import heapq
from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple


class OracleError(Exception):
    pass


class OOMError(OracleError):
    pass


class LockError(OracleError):
    pass


class SlotError(OracleError):
    pass


class NodeError(OracleError):
    pass


POLICIES = ("lru", "lfu", "slru", "fifo", "mru", "filo", "priority")


class Node:
    __slots__ = ("id", "parent", "children", "key", "value", "lock_ref", "last", "hits", "created", "priority")

    def __init__(self, nid: int, parent: Optional["Node"], key: List[int], value: List[int],
                 lock_ref: int, last: int, hits: int = 0, created: int = 0, priority: int = 0):
        self.id = nid
        self.parent = parent
        self.children: Dict[int, "Node"] = {}
        self.key = key
        self.value = value
        self.lock_ref = lock_ref
        self.last = last
        self.hits = hits
        self.created = created
        self.priority = priority


def evict_key(policy: str, n: Node):
    if policy == "lru":
        return (n.last, n.id)
    if policy == "mru":
        return (-n.last, n.id)
    if policy == "fifo":
        return (n.created, n.id)
    if policy == "filo":
        return (-n.created, n.id)
    if policy == "lfu":
        return (n.hits, n.last, n.id)
    if policy == "slru":
        return (1 if n.hits >= 2 else 0, n.last, n.id)
    if policy == "priority":
        return (n.priority, n.last, n.id)
    raise ValueError(policy)


def lcp(a: Sequence[int], b: Sequence[int]) -> int:
    """Length of the longest common prefix of two token runs."""
    n = min(len(a), len(b))
    i = 0
    while i < n and a[i] == b[i]:
        i += 1
    return i


class OracleTree:
    def __init__(self, pool_slots: int, free_order: Optional[Sequence[int]] = None, policy: str = "lru"):
        if policy not in POLICIES:
            raise OracleError(f"unknown eviction policy {policy}")
        self.policy = policy
        self.pool_slots = int(pool_slots)
        order = list(range(pool_slots)) if free_order is None else [int(s) for s in free_order]
        if len(set(order)) != len(order) or any(s < 0 or s >= pool_slots for s in order):
            raise SlotError("bad initial free order")
        self.capacity = len(order)
        self.free = deque(order)
        self._is_free = set(order)
        self.root = Node(0, None, [], [], 1, 0)
        self.nodes: Dict[int, Node] = {0: self.root}
        self.clock = 0
        self.next_id = 1
        self.evictable = 0
        self.protected = 0
        self.evlog: List[Tuple[int, List[int]]] = []

    # -- helpers -----------------------------------------------------------------
    def _node(self, nid: int) -> Node:
        n = self.nodes.get(int(nid))
        if n is None:
            raise NodeError(f"node {nid} is not live")
        return n

    def _split(self, child: Node, k: int) -> Node:
        """Cut ``child`` after its first k tokens; return the new upper node."""
        parent = child.parent
        upper = Node(self.next_id, parent, child.key[:k], child.value[:k], child.lock_ref, self.clock,
                     child.hits, child.created, child.priority)
        self.next_id += 1
        self.nodes[upper.id] = upper
        child.key = child.key[k:]
        child.value = child.value[k:]
        child.parent = upper
        upper.children[child.key[0]] = child
        parent.children[upper.key[0]] = upper
        return upper

    # -- public operations ----------------------------------------------------------
    def match(self, key: Sequence[int]) -> Tuple[int, List[int], int]:
        """Longest cached prefix of ``key``: (length, its slots, id of the node ending it)."""
        self.clock += 1
        key = [int(t) for t in key]
        node = self.root
        slots: List[int] = []
        while key and key[0] in node.children:
            child = node.children[key[0]]
            child.last = self.clock
            k = lcp(child.key, key)
            if k < len(child.key):
                upper = self._split(child, k)
                upper.hits += 1
                slots.extend(upper.value)
                node = upper
                break
            child.hits += 1
            slots.extend(child.value)
            node = child
            key = key[k:]
        return len(slots), slots, node.id

    def peek(self, key: Sequence[int]) -> int:
        """Length of the cached prefix of ``key``; changes nothing (no split, no stamp)."""
        key = [int(t) for t in key]
        node = self.root
        m = 0
        while key and key[0] in node.children:
            child = node.children[key[0]]
            k = lcp(child.key, key)
            m += k
            if k < len(child.key):
                break
            node = child
            key = key[k:]
        return m

    def insert(self, key: Sequence[int], value: Sequence[int], priority: int = 0) -> Tuple[int, int]:
        """Insert key -> value; return (already-cached length, id of the node ending the key)."""
        if len(key) != len(value):
            raise OracleError("key and value lengths differ")
        self.clock += 1
        key = [int(t) for t in key]
        value = [int(s) for s in value]
        node = self.root
        total = 0
        while key and key[0] in node.children:
            child = node.children[key[0]]
            child.last = self.clock
            k = lcp(child.key, key)
            total += k
            key = key[k:]
            value = value[k:]
            if k < len(child.key):
                node = self._split(child, k)
                node.priority = max(node.priority, priority)
                break
            child.priority = max(child.priority, priority)
            node = child
        if key:
            leaf = Node(self.next_id, node, key, value, 0, self.clock, 0, self.clock, priority)
            self.next_id += 1
            self.nodes[leaf.id] = leaf
            node.children[key[0]] = leaf
            self.evictable += len(key)
            node = leaf
        return total, node.id

    def inc_lock(self, nid: int) -> None:
        node = self._node(nid)
        while node is not self.root:
            if node.lock_ref == 0:
                self.evictable -= len(node.key)
                self.protected += len(node.key)
            node.lock_ref += 1
            node = node.parent

    def dec_lock(self, nid: int) -> None:
        node = self._node(nid)
        if node is not self.root and node.lock_ref == 0:
            raise LockError(f"node {nid} is not locked")
        while node is not self.root:
            if node.lock_ref == 1:
                self.evictable += len(node.key)
                self.protected -= len(node.key)
            node.lock_ref -= 1
            node = node.parent

    def evict(self, num_tokens: int) -> int:
        heap = [(evict_key(self.policy, n), n.id) for n in self.nodes.values()
                if n is not self.root and not n.children and n.lock_ref == 0]
        heapq.heapify(heap)
        evicted = 0
        while evicted < num_tokens and heap:
            _, nid = heapq.heappop(heap)
            x = self.nodes[nid]
            for s in x.value:
                self.free.append(s)
                self._is_free.add(s)
            self.evlog.append((x.id, list(x.value)))
            evicted += len(x.value)
            self.evictable -= len(x.key)
            parent = x.parent
            del parent.children[x.key[0]]
            del self.nodes[x.id]
            if parent is not self.root and not parent.children and parent.lock_ref == 0:
                heapq.heappush(heap, (evict_key(self.policy, parent), parent.id))
        return evicted

    def alloc(self, n: int) -> List[int]:
        if n < 0:
            raise OracleError("negative allocation")
        if len(self.free) < n:
            self.evict(n - len(self.free))
        if len(self.free) < n:
            raise OOMError(f"need {n} slots, {len(self.free)} free after eviction")
        out = [self.free.popleft() for _ in range(n)]
        for s in out:
            self._is_free.discard(s)
        return out

    def free_slots(self, slots: Sequence[int]) -> None:
        slots = [int(s) for s in slots]
        seen = set()
        for s in slots:
            if s < 0 or s >= self.pool_slots or s in self._is_free or s in seen:
                raise SlotError(f"slot {s} out of range or already free")
            seen.add(s)
        for s in slots:
            self.free.append(s)
            self._is_free.add(s)

    def take_evlog(self) -> List[Tuple[int, List[int]]]:
        out, self.evlog = self.evlog, []
        return out

    # -- introspection (for tests) ------------------------------------------------
    def cached_tokens(self) -> int:
        return sum(len(n.key) for n in self.nodes.values() if n is not self.root)

    def dump(self) -> List[Tuple[int, int, int, int, Tuple[int, ...], Tuple[int, ...]]]:
        """Live non-root nodes as (id, parent id, lock_ref, last, key, value), by id."""
        out = []
        for nid in sorted(self.nodes):
            n = self.nodes[nid]
            if n is self.root:
                continue
            out.append((n.id, n.parent.id, n.lock_ref, n.last, tuple(n.key), tuple(n.value)))
        return out

    def dump_stats(self) -> List[Tuple[int, int, int, int]]:
        """Live non-root nodes as (id, hit count, created, priority), by id."""
        return [(n.id, n.hits, n.created, n.priority) for nid, n in sorted(self.nodes.items()) if n is not self.root]

    def path_tokens(self, nid: int) -> List[int]:
        node = self._node(nid)
        parts = []
        while node is not self.root:
            parts.append(node.key)
            node = node.parent
        return [t for p in reversed(parts) for t in p]
