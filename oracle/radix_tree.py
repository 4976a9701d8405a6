"""Oracle radix tree over token ids with a token-granular slot pool.  TEST INFRASTRUCTURE ONLY.

What the cache holds, in the terms of the pages rather than of any code listing:
- a set of cached token sequences, closed under prefixes, each cached position carrying one
  KV slot (one slot per token: the radix-cache walkthrough page "[SGLang] RadixAttention:
  Radix Tree 기반 프리픽스 캐싱의 핵심", sections "Radix Tree 구조도" and "핵심 자료구조:
  TreeNode");
- that set cut into runs of consecutive positions ("nodes"): a node is where the tree keeps
  its lock reference, access time and the other eviction fields, and it is the unit of
  eviction (section "Eviction 전략").

Here the set is stored as a token trie, one vertex per cached position (so a prefix match
is plainly the longest common prefix of the key with the cached sequences, the matching
formula of the RadixAttention explainer "論文解説: Efficiently Programming Large Language
Models using SGLang", section "プレフィックスマッチングアルゴリズム"), and a node is a list of
vertices.  Operations, stated as what they do to that set:
- match(key): m = longest common prefix of key with the cached set.  If position m - 1 lies
  inside a node rather than at its end, that node is cut there into an upper part (positions
  up to m - 1, a new id) and a lower part (the rest, the old id), "노드 분할"; both parts and
  every other node holding a matched position take the call's access time; the nodes holding
  a matched position count one more hit.  Result: m, the slots of positions 0..m-1, and the
  node ending position m - 1 (0, the root, when m = 0) ("프리픽스 매칭").
- insert(key, slots): the same cut at the cached length m and the same access stamps; the
  positions m.. of key become one new node with the given slots; the cached slots of 0..m-1
  stay (the caller's slots for them are duplicates it frees) ("삽입").
- inc_lock / dec_lock(node): +-1 on the node and every node above it on its path to the
  root; a node's tokens count as protected while its lock is above 0 ("참조 카운트").
- evict(n): while fewer than n tokens are freed, look at every node that is unlocked and
  has nothing cached below it, remove the one with the smallest policy key, and hand its
  slots back ("Eviction 전략").

Readings where the pages leave a step open (each is listed in the design notes):
- access time is a logical clock, +1 per match or insert call; every node holding a
  position the call walked over, both parts of a cut and a new node get the call's value;
- insert cuts a node at the cached length exactly like match does (the page elides that
  branch) and stamps the nodes it walks over;
- eviction keys end in the node id, ascending; ids come from a creation counter (the upper
  part of a cut takes a new id, the lower part keeps its id);
- eviction removes whole nodes and stops once at least the requested number of tokens is
  freed;
- the free list is first-in first-out: allocation pops from the head, frees append to the
  tail in the order given (a removed node's slots in position order);
- allocation evicts (requested - free) tokens when the free list is short, then fails with
  OOM if it is still short.

Eviction policies (the page names lru, lfu, slru, fifo, mru, filo and priority as strategy
objects without their keys; these are the readings taken):
- lru (default): (last access, id)            - mru: (-last access, id)
- fifo: (created, id)                          - filo: (-created, id)
- lfu: (hit count, last access, id)            - priority: (priority, last access, id)
- slru: (protected, last access, id), protected = hit count >= 2 (probationary first)
Node fields behind them: hit count = number of match calls that reused at least one of the
node's positions (the upper part of a cut starts from the old count and takes the call's
hit, the lower part keeps the old count); created = clock of the insert that first cached
the node's first position (both parts of a cut keep it); priority = max of the priorities of
the inserts that walked over one of the node's positions or created it (both parts of a cut
keep the old value; only the part holding walked positions is raised).
"""
from __future__ import annotations

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
    """A run of consecutive cached positions (trie vertices) and its cache fields."""
    __slots__ = ("id", "verts", "lock_ref", "last", "hits", "created", "priority")

    def __init__(self, nid: int, verts: List[int], lock_ref: int, last: int, hits: int = 0, created: int = 0,
                 priority: int = 0):
        self.id = nid
        self.verts = verts
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


ROOT_VERTEX = 0


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
        # trie of cached positions: vertex 0 is the empty prefix
        self.v_tok: List[int] = [-1]
        self.v_par: List[int] = [-1]
        self.v_slot: List[int] = [-1]
        self.v_node: List[int] = [0]
        self.v_nchild: List[int] = [0]
        self.edge: Dict[Tuple[int, int], int] = {}        # (parent vertex, token) -> vertex
        self.root = Node(0, [ROOT_VERTEX], 1, 0)
        self.nodes: Dict[int, Node] = {0: self.root}
        self.clock = 0
        self.next_id = 1
        self.evictable = 0
        self.protected = 0
        self.evlog: List[Tuple[int, List[int]]] = []

    # -- the cached set ------------------------------------------------------------
    def _walk(self, key: Sequence[int]) -> List[int]:
        """Vertices of the longest cached prefix of key, in position order."""
        path = []
        v = ROOT_VERTEX
        for tok in key:
            w = self.edge.get((v, int(tok)))
            if w is None:
                break
            path.append(w)
            v = w
        return path

    def _node(self, nid: int) -> Node:
        n = self.nodes.get(int(nid))
        if n is None:
            raise NodeError(f"node {nid} is not live")
        return n

    def _parent(self, n: Node) -> Node:
        return self.nodes[self.v_node[self.v_par[n.verts[0]]]]

    def _nodes_over(self, path: List[int]) -> List[Node]:
        """Distinct nodes holding the positions of path, root side first."""
        out: List[Node] = []
        for v in path:
            n = self.nodes[self.v_node[v]]
            if not out or out[-1] is not n:
                out.append(n)
        return out

    def _cut_after(self, v: int) -> None:
        """Make vertex v the last position of its node: the positions up to v become a new
        upper node (new id, the old node's fields, this call's access time)."""
        low = self.nodes[self.v_node[v]]
        i = low.verts.index(v)
        if i == len(low.verts) - 1:
            return
        up = Node(self.next_id, low.verts[:i + 1], low.lock_ref, self.clock, low.hits, low.created, low.priority)
        self.next_id += 1
        self.nodes[up.id] = up
        low.verts = low.verts[i + 1:]
        for u in up.verts:
            self.v_node[u] = up.id

    def _walk_and_cut(self, key: Sequence[int]) -> List[int]:
        """The common step of match and insert: stamp the nodes over the cached prefix and cut
        the one the prefix ends inside of."""
        path = self._walk(key)
        for n in self._nodes_over(path):
            n.last = self.clock
        if path:
            self._cut_after(path[-1])
        return path

    def _add_vertices(self, parent: int, toks: Sequence[int], slots: Sequence[int], nid: int) -> List[int]:
        out = []
        for t, s in zip(toks, slots):
            w = len(self.v_tok)
            self.v_tok.append(int(t))
            self.v_par.append(parent)
            self.v_slot.append(int(s))
            self.v_node.append(nid)
            self.v_nchild.append(0)
            self.edge[(parent, int(t))] = w
            self.v_nchild[parent] += 1
            out.append(w)
            parent = w
        return out

    def _is_leaf(self, n: Node) -> bool:
        return self.v_nchild[n.verts[-1]] == 0

    def _remove(self, n: Node) -> None:
        for w in reversed(n.verts):
            p = self.v_par[w]
            del self.edge[(p, self.v_tok[w])]
            self.v_nchild[p] -= 1
            self.v_node[w] = -1
        del self.nodes[n.id]

    # -- public operations ----------------------------------------------------------
    def match(self, key: Sequence[int]) -> Tuple[int, List[int], int]:
        """Longest cached prefix of ``key``: (length, its slots, id of the node ending it)."""
        self.clock += 1
        path = self._walk_and_cut(key)
        for n in self._nodes_over(path):
            n.hits += 1
        end = self.v_node[path[-1]] if path else 0
        return len(path), [self.v_slot[v] for v in path], end

    def peek(self, key: Sequence[int]) -> int:
        """Length of the cached prefix of ``key``; changes nothing (no cut, no stamp)."""
        return len(self._walk(key))

    def insert(self, key: Sequence[int], value: Sequence[int], priority: int = 0) -> Tuple[int, int]:
        """Cache key -> value; return (already-cached length, id of the node ending the key)."""
        if len(key) != len(value):
            raise OracleError("key and value lengths differ")
        self.clock += 1
        key = [int(t) for t in key]
        path = self._walk_and_cut(key)
        for n in self._nodes_over(path):
            n.priority = max(n.priority, priority)
        m = len(path)
        if m == len(key):
            return m, (self.v_node[path[-1]] if path else 0)
        leaf = Node(self.next_id, [], 0, self.clock, 0, self.clock, priority)
        self.next_id += 1
        self.nodes[leaf.id] = leaf
        leaf.verts = self._add_vertices(path[-1] if path else ROOT_VERTEX, key[m:], list(value)[m:], leaf.id)
        self.evictable += len(key) - m
        return m, leaf.id

    def _path_to_root(self, n: Node):
        while n is not self.root:
            yield n
            n = self._parent(n)

    def inc_lock(self, nid: int) -> None:
        for n in self._path_to_root(self._node(nid)):
            if n.lock_ref == 0:
                self.evictable -= len(n.verts)
                self.protected += len(n.verts)
            n.lock_ref += 1

    def dec_lock(self, nid: int) -> None:
        node = self._node(nid)
        if node is not self.root and node.lock_ref == 0:
            raise LockError(f"node {nid} is not locked")
        for n in self._path_to_root(node):
            if n.lock_ref == 1:
                self.evictable += len(n.verts)
                self.protected -= len(n.verts)
            n.lock_ref -= 1

    def evict(self, num_tokens: int) -> int:
        evicted = 0
        # the unlocked nodes with nothing cached below them; a parent joins once its last
        # child is gone
        cands = [n for n in self.nodes.values() if n is not self.root and n.lock_ref == 0 and self._is_leaf(n)]
        while evicted < num_tokens and cands:
            x = min(cands, key=lambda n: evict_key(self.policy, n))
            cands.remove(x)
            parent = self._parent(x)
            slots = [self.v_slot[w] for w in x.verts]
            for s in slots:
                self.free.append(s)
                self._is_free.add(s)
            self.evlog.append((x.id, slots))
            evicted += len(slots)
            self.evictable -= len(slots)
            self._remove(x)
            if parent is not self.root and parent.lock_ref == 0 and self._is_leaf(parent):
                cands.append(parent)
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
        return sum(len(n.verts) for n in self.nodes.values() if n is not self.root)

    def dump(self) -> List[Tuple[int, int, int, int, Tuple[int, ...], Tuple[int, ...]]]:
        """Live non-root nodes as (id, parent id, lock_ref, last, key, value), by id."""
        out = []
        for nid in sorted(self.nodes):
            n = self.nodes[nid]
            if n is self.root:
                continue
            out.append((n.id, self._parent(n).id, n.lock_ref, n.last, tuple(self.v_tok[w] for w in n.verts),
                        tuple(self.v_slot[w] for w in n.verts)))
        return out

    def dump_stats(self) -> List[Tuple[int, int, int, int]]:
        """Live non-root nodes as (id, hit count, created, priority), by id."""
        return [(n.id, n.hits, n.created, n.priority) for nid, n in sorted(self.nodes.items()) if n is not self.root]

    def path_tokens(self, nid: int) -> List[int]:
        """Token sequence from the root to the end of node nid."""
        n = self._node(nid)
        out = []
        v = n.verts[-1]
        while v != ROOT_VERTEX:
            out.append(self.v_tok[v])
            v = self.v_par[v]
        return out[::-1]
