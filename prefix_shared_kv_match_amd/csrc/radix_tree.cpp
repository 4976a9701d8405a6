// Host radix tree over token ids with a token-granular KV slot allocator.
//
// Semantics follow the radix-cache walkthrough page "[SGLang] RadixAttention: Radix
// Tree 기반 프리픽스 캐싱의 핵심": nodes hold a run of tokens (key) and one KV slot per
// token (value); children are keyed by their first token; match walks whole children
// and splits a partially matched one (sections "프리픽스 매칭", "노드 분할"); insert
// walks the same way and hangs the rest as a new evictable leaf (section "삽입");
// lock references run up to the root and move tokens between the evictable and
// protected counts (section "참조 카운트"); eviction pops unlocked leaves in LRU order
// and pushes parents that become unlocked leaves (section "Eviction 전략").
//
// Where the page leaves a step open this code takes these readings:
//  - access time is a logical clock advanced once per match / insert call; every node
//    visited in the call, both halves of a split and a new leaf get that value;
//  - insert splits a partially matched node like match does;
//  - the eviction order key is (access time, node id) ascending; a split's upper node
//    takes a fresh id and the lower part keeps its id;
//  - eviction removes whole leaves and stops once >= the requested tokens are freed;
//  - the free list is FIFO: allocate from the head, free/evict to the tail;
//  - allocation evicts (n - free) tokens on shortfall, then reports OOM.
//  - the page's policy family (lru, lfu, slru, fifo, mru, filo, priority) are ascending
//    heap keys ending in the node id: lru (last access), mru (-last access), fifo / filo
//    (+-creation clock), lfu (hit count, last access), priority (priority, last access), slru
//    (protected = hit count >= 2, last access).  Hit count = match calls that reused a token of
//    the node (a split's upper half takes the old count + 1); creation clock and priority are
//    inherited by a split's upper half; priority is the max over inserts through the node.
//
// Storage: nodes live in a vector indexed by id (ids are never reused); a compact list
// of live ids keeps the eviction scan proportional to the live tree.  Slot ownership
// is tracked per slot so that double frees and foreign slots are rejected.

#include <algorithm>
#include <cstring>
#include <queue>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace {

enum SlotState : uint8_t { kUnavailable = 0, kFree = 1, kInFlight = 2, kCached = 3, kMark = 4 };

struct Node {
  int64_t parent = -1;
  std::vector<int32_t> key;
  std::vector<int32_t> value;
  std::unordered_map<int32_t, int64_t> children;
  int64_t lock_ref = 0;
  int64_t last = 0;
  int64_t hits = 0;
  int64_t created = 0;
  int64_t priority = 0;
  int64_t live_pos = -1;  // index in Tree::live, -1 when dead
};

enum Policy : int32_t { kLRU = 0, kLFU = 1, kSLRU = 2, kFIFO = 3, kMRU = 4, kFILO = 5, kPriority = 6 };

struct EvictKey {
  int64_t a, b, id;
  bool operator>(const EvictKey& o) const {
    if (a != o.a) return a > o.a;
    if (b != o.b) return b > o.b;
    return id > o.id;
  }
};

inline EvictKey evict_key(int32_t policy, const Node& n, int64_t id) {
  switch (policy) {
    case kMRU: return EvictKey{-n.last, 0, id};
    case kFIFO: return EvictKey{n.created, 0, id};
    case kFILO: return EvictKey{-n.created, 0, id};
    case kLFU: return EvictKey{n.hits, n.last, id};
    case kSLRU: return EvictKey{n.hits >= 2 ? 1 : 0, n.last, id};
    case kPriority: return EvictKey{n.priority, n.last, id};
    default: return EvictKey{n.last, 0, id};
  }
}

// Length of the common prefix of a[0..na) and b[0..nb): whole 64-token blocks are compared
// with memcmp (vectorised in the C library), the first differing block token by token.
inline int64_t lcp(const int32_t* a, int64_t na, const int32_t* b, int64_t nb) {
  const int64_t n = std::min(na, nb);
  constexpr int64_t kBlock = 64;
  int64_t i = 0;
  while (i + kBlock <= n && std::memcmp(a + i, b + i, kBlock * sizeof(int32_t)) == 0) i += kBlock;
  while (i < n && a[i] == b[i]) ++i;
  return i;
}

}  // namespace

struct rt_tree {
  int32_t policy = kLRU;
  int64_t num_slots = 0;
  std::vector<uint8_t> state;      // per slot
  std::vector<int32_t> ring;       // FIFO free list storage
  int64_t head = 0, count = 0;
  std::vector<Node> nodes;         // index = node id, 0 = root
  std::vector<int64_t> live;       // live non-root node ids
  int64_t clock = 0;
  int64_t evictable = 0, protected_ = 0;
  std::vector<int64_t> log_ids, log_lens;
  std::vector<int32_t> log_slots;
  bool log_on = true;

  bool is_live(int64_t id) const {
    return id == 0 || (id > 0 && id < (int64_t)nodes.size() && nodes[id].live_pos >= 0);
  }

  // the free list is a ring of ring.size() entries (head < ring.size(), count <= ring.size());
  // index arithmetic wraps with one compare instead of a division
  void push_free(int32_t s) {
    int64_t i = head + count;
    if (i >= (int64_t)ring.size()) i -= (int64_t)ring.size();
    ring[i] = s;
    ++count;
    state[s] = kFree;
  }
  int32_t pop_free() {
    int32_t s = ring[head];
    if (++head == (int64_t)ring.size()) head = 0;
    --count;
    state[s] = kInFlight;
    return s;
  }

  int64_t new_node() {
    nodes.emplace_back();
    int64_t id = (int64_t)nodes.size() - 1;
    nodes[id].live_pos = (int64_t)live.size();
    live.push_back(id);
    return id;
  }
  void kill(int64_t id) {
    Node& x = nodes[id];
    int64_t pos = x.live_pos;
    int64_t moved = live.back();
    live[pos] = moved;
    nodes[moved].live_pos = pos;
    live.pop_back();
    x.live_pos = -1;
    std::vector<int32_t>().swap(x.key);
    std::vector<int32_t>().swap(x.value);
    std::unordered_map<int32_t, int64_t>().swap(x.children);
  }

  // Cut node c after its first k tokens; returns the new upper node's id.
  int64_t split(int64_t c, int64_t k) {
    int64_t up = new_node();
    Node& U = nodes[up];
    Node& C = nodes[c];
    U.parent = C.parent;
    U.lock_ref = C.lock_ref;
    U.last = clock;
    U.hits = C.hits;
    U.created = C.created;
    U.priority = C.priority;
    U.key.assign(C.key.begin(), C.key.begin() + k);
    U.value.assign(C.value.begin(), C.value.begin() + k);
    C.key.erase(C.key.begin(), C.key.begin() + k);
    C.value.erase(C.value.begin(), C.value.begin() + k);
    C.parent = up;
    U.children[C.key[0]] = c;
    nodes[U.parent].children[U.key[0]] = up;
    return up;
  }

  // Read-only walk: length of the cached prefix of key (no stamps, no splits).
  int64_t peek(const int32_t* key, int64_t n) const {
    int64_t cur = 0, pos = 0;
    while (pos < n) {
      const Node& N = nodes[cur];
      auto it = N.children.find(key[pos]);
      if (it == N.children.end()) break;
      const Node& C = nodes[it->second];
      int64_t k = lcp(C.key.data(), (int64_t)C.key.size(), key + pos, n - pos);
      pos += k;
      if (k < (int64_t)C.key.size()) break;
      cur = it->second;
    }
    return pos;
  }

  int64_t match(const int32_t* key, int64_t n, int32_t* out, int64_t* out_last) {
    ++clock;
    int64_t cur = 0, pos = 0;
    while (pos < n) {
      auto it = nodes[cur].children.find(key[pos]);
      if (it == nodes[cur].children.end()) break;
      int64_t c = it->second;
      nodes[c].last = clock;
      int64_t klen = (int64_t)nodes[c].key.size();
      int64_t k = lcp(nodes[c].key.data(), klen, key + pos, n - pos);
      if (k < klen) {
        int64_t up = split(c, k);
        ++nodes[up].hits;
        std::memcpy(out + pos, nodes[up].value.data(), sizeof(int32_t) * k);
        pos += k;
        cur = up;
        break;
      }
      ++nodes[c].hits;
      std::memcpy(out + pos, nodes[c].value.data(), sizeof(int32_t) * k);
      pos += k;
      cur = c;
    }
    *out_last = cur;
    return pos;
  }

  // Checks that slots[0..n) are distinct and in flight.
  int check_in_flight(const int32_t* slots, int64_t n) {
    int64_t i = 0;
    int rc = PKV_OK;
    for (; i < n; ++i) {
      int32_t s = slots[i];
      if (s < 0 || s >= num_slots || state[s] != kInFlight) {
        rc = pkv::fail(PKV_ERR_SLOT, "slot %d is out of range, repeated, or not in flight", s);
        break;
      }
      state[s] = kMark;
    }
    for (int64_t j = 0; j < i; ++j) state[slots[j]] = kInFlight;
    return rc;
  }

  int64_t insert(const int32_t* key, const int32_t* slots, int64_t n, int64_t* out_last, int64_t priority = 0) {
    int64_t m = peek(key, n);
    int rc = check_in_flight(slots + m, n - m);
    if (rc < 0) return rc;
    ++clock;
    int64_t cur = 0, pos = 0;
    while (pos < n) {
      auto it = nodes[cur].children.find(key[pos]);
      if (it == nodes[cur].children.end()) break;
      int64_t c = it->second;
      nodes[c].last = clock;
      int64_t klen = (int64_t)nodes[c].key.size();
      int64_t k = lcp(nodes[c].key.data(), klen, key + pos, n - pos);
      pos += k;
      if (k < klen) {
        cur = split(c, k);
        nodes[cur].priority = std::max(nodes[cur].priority, priority);
        break;
      }
      nodes[c].priority = std::max(nodes[c].priority, priority);
      cur = c;
    }
    if (pos != m) return pkv::fail(PKV_ERR_INTERNAL, "insert walk disagrees with peek (%lld vs %lld)",
                                   (long long)pos, (long long)m);
    if (pos < n) {
      int64_t leaf = new_node();
      Node& L = nodes[leaf];
      L.parent = cur;
      L.key.assign(key + pos, key + n);
      L.value.assign(slots + pos, slots + n);
      L.last = clock;
      L.created = clock;
      L.priority = priority;
      nodes[cur].children[key[pos]] = leaf;
      evictable += n - pos;
      for (int64_t i = pos; i < n; ++i) state[slots[i]] = kCached;
      cur = leaf;
    }
    *out_last = cur;
    return m;
  }

  // Tokens from the root to the end of node id (the node's depth in tokens).
  int64_t depth(int64_t id) const {
    int64_t d = 0;
    for (; id > 0; id = nodes[id].parent) d += (int64_t)nodes[id].key.size();
    return d;
  }

  // insert() for a key whose first m tokens are known to be the cached path ending at node a
  // (a match result or a prompt's end node, locked so the path cannot have changed).  The
  // root walk of insert() would visit exactly the nodes from the root down to a, so they are
  // stamped (and their priorities raised) through the parent links, and the walk resumes at
  // a: the same tree, clock and result as insert(key, ...), without re-reading the first m
  // tokens.
  int64_t insert_below(int64_t a, int64_t m, const int32_t* key, const int32_t* slots, int64_t n, int64_t* out_last,
                       int64_t priority = 0) {
    // tokens cached below a (normally none after a match)
    int64_t more = 0;
    {
      int64_t cur = a, pos = m;
      while (pos < n) {
        const Node& N = nodes[cur];
        auto it = N.children.find(key[pos]);
        if (it == N.children.end()) break;
        const Node& C = nodes[it->second];
        const int64_t k = lcp(C.key.data(), (int64_t)C.key.size(), key + pos, n - pos);
        pos += k;
        if (k < (int64_t)C.key.size()) break;
        cur = it->second;
      }
      more = pos - m;
    }
    int rc = check_in_flight(slots + m + more, n - m - more);
    if (rc < 0) return rc;
    ++clock;
    for (int64_t id = a; id > 0; id = nodes[id].parent) {
      nodes[id].last = clock;
      nodes[id].priority = std::max(nodes[id].priority, priority);
    }
    int64_t cur = a, pos = m;
    while (pos < n) {
      auto it = nodes[cur].children.find(key[pos]);
      if (it == nodes[cur].children.end()) break;
      int64_t c = it->second;
      nodes[c].last = clock;
      int64_t klen = (int64_t)nodes[c].key.size();
      int64_t k = lcp(nodes[c].key.data(), klen, key + pos, n - pos);
      pos += k;
      if (k < klen) {
        cur = split(c, k);
        nodes[cur].priority = std::max(nodes[cur].priority, priority);
        break;
      }
      nodes[c].priority = std::max(nodes[c].priority, priority);
      cur = c;
    }
    if (pos < n) {
      int64_t leaf = new_node();
      Node& L = nodes[leaf];
      L.parent = cur;
      L.key.assign(key + pos, key + n);
      L.value.assign(slots + pos, slots + n);
      L.last = clock;
      L.created = clock;
      L.priority = priority;
      nodes[cur].children[key[pos]] = leaf;
      evictable += n - pos;
      for (int64_t i = pos; i < n; ++i) state[slots[i]] = kCached;
      cur = leaf;
    }
    *out_last = cur;
    return m + more;
  }

  int inc_lock(int64_t id) {
    if (!is_live(id)) return pkv::fail(PKV_ERR_NODE, "node %lld is not live", (long long)id);
    while (id != 0) {
      Node& x = nodes[id];
      if (x.lock_ref == 0) {
        evictable -= (int64_t)x.key.size();
        protected_ += (int64_t)x.key.size();
      }
      ++x.lock_ref;
      id = x.parent;
    }
    return PKV_OK;
  }

  int dec_lock(int64_t id) {
    if (!is_live(id)) return pkv::fail(PKV_ERR_NODE, "node %lld is not live", (long long)id);
    if (id != 0 && nodes[id].lock_ref == 0)
      return pkv::fail(PKV_ERR_LOCK, "node %lld is not locked", (long long)id);
    while (id != 0) {
      Node& x = nodes[id];
      if (x.lock_ref == 1) {
        evictable += (int64_t)x.key.size();
        protected_ -= (int64_t)x.key.size();
      }
      --x.lock_ref;
      id = x.parent;
    }
    return PKV_OK;
  }

  int64_t evict(int64_t num_tokens) {
    std::priority_queue<EvictKey, std::vector<EvictKey>, std::greater<EvictKey>> heap;
    for (int64_t id : live) {
      const Node& x = nodes[id];
      if (x.children.empty() && x.lock_ref == 0) heap.push(evict_key(policy, x, id));
    }
    int64_t evicted = 0;
    while (evicted < num_tokens && !heap.empty()) {
      int64_t id = heap.top().id;
      heap.pop();
      Node& x = nodes[id];
      for (int32_t s : x.value) push_free(s);
      if (log_on) {
        log_ids.push_back(id);
        log_lens.push_back((int64_t)x.value.size());
        log_slots.insert(log_slots.end(), x.value.begin(), x.value.end());
      }
      evicted += (int64_t)x.value.size();
      evictable -= (int64_t)x.key.size();
      int64_t p = x.parent;
      nodes[p].children.erase(x.key[0]);
      kill(id);
      const Node& P = nodes[p];
      if (p != 0 && P.children.empty() && P.lock_ref == 0) heap.push(evict_key(policy, P, p));
    }
    return evicted;
  }

  int64_t alloc(int64_t n, int32_t* out) {
    if (n < 0) return pkv::fail(PKV_ERR_INVAL, "negative allocation");
    if (count < n) evict(n - count);
    if (count < n)
      return pkv::fail(PKV_ERR_OOM, "need %lld slots, %lld free after eviction", (long long)n, (long long)count);
    for (int64_t i = 0; i < n; ++i) out[i] = pop_free();
    return n;
  }

  int free_slots(const int32_t* slots, int64_t n) {
    int rc = check_in_flight(slots, n);
    if (rc < 0) return rc;
    for (int64_t i = 0; i < n; ++i) push_free(slots[i]);
    return PKV_OK;
  }
};

namespace {

template <class F>
auto guard(F&& f) -> decltype(f()) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return pkv::fail(PKV_ERR_INTERNAL, "host allocation failed");
  } catch (...) {
    return pkv::fail(PKV_ERR_INTERNAL, "unexpected C++ exception");
  }
}

}  // namespace

extern "C" {

int rt_create(int64_t num_slots, const int32_t* free_order, int64_t n_free, rt_tree** out) {
  return rt_create_policy(num_slots, free_order, n_free, kLRU, out);
}

int rt_create_policy(int64_t num_slots, const int32_t* free_order, int64_t n_free, int32_t policy, rt_tree** out) {
  return guard([&]() -> int {
    if (policy < kLRU || policy > kPriority) return pkv::fail(PKV_ERR_INVAL, "unknown eviction policy %d", policy);
    if (!out) return pkv::fail(PKV_ERR_INVAL, "out is null");
    *out = nullptr;
    if (num_slots <= 0 || num_slots > INT32_MAX) return pkv::fail(PKV_ERR_INVAL, "num_slots out of range");
    if (!free_order) n_free = num_slots;
    if (n_free < 0 || n_free > num_slots) return pkv::fail(PKV_ERR_INVAL, "n_free out of range");
    rt_tree* t = new rt_tree();
    t->num_slots = num_slots;
    t->state.assign((size_t)num_slots, kUnavailable);
    t->ring.assign((size_t)std::max<int64_t>(n_free, 1), 0);
    for (int64_t i = 0; i < n_free; ++i) {
      int32_t s = free_order ? free_order[i] : (int32_t)i;
      if (s < 0 || s >= num_slots || t->state[s] != kUnavailable) {
        delete t;
        return pkv::fail(PKV_ERR_SLOT, "free_order[%lld] = %d is out of range or repeated", (long long)i, s);
      }
      t->push_free(s);
    }
    t->nodes.emplace_back();  // root
    t->nodes[0].lock_ref = 1;
    t->policy = policy;
    *out = t;
    return PKV_OK;
  });
}

void rt_destroy(rt_tree* t) { delete t; }

int64_t rt_match_prefix(rt_tree* t, const int32_t* key, int64_t n, int32_t* out_slots, rt_node* out_last) {
  return guard([&]() -> int64_t {
    if (!t || !out_last || n < 0 || (n > 0 && (!key || !out_slots)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_match_prefix");
    return t->match(key, n, out_slots, out_last);
  });
}

int64_t rt_insert(rt_tree* t, const int32_t* key, const int32_t* slots, int64_t n, rt_node* out_last) {
  return rt_insert_priority(t, key, slots, n, 0, out_last);
}

int64_t rt_insert_priority(rt_tree* t, const int32_t* key, const int32_t* slots, int64_t n, int32_t priority,
                           rt_node* out_last) {
  return guard([&]() -> int64_t {
    if (!t || !out_last || n < 0 || (n > 0 && (!key || !slots)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_insert");
    return t->insert(key, slots, n, out_last, priority);
  });
}

int64_t rt_peek_prefix(const rt_tree* t, const int32_t* key, int64_t n) {
  if (!t || n < 0 || (n > 0 && !key)) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_peek_prefix");
  return t->peek(key, n);
}

int rt_schedule_longest_prefix(const rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                               int32_t* order, int64_t* match_lens) {
  return guard([&]() -> int {
    if (!t || num_reqs < 0 || (num_reqs > 0 && (!tokens || !tok_indptr || !order)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_schedule_longest_prefix");
    std::vector<int64_t> m((size_t)num_reqs);
    for (int32_t r = 0; r < num_reqs; ++r) {
      const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
      if (L < 0) return pkv::fail(PKV_ERR_INVAL, "request %d has a negative length", r);
      m[r] = t->peek(tokens + tok_indptr[r], L);
      order[r] = r;
    }
    std::stable_sort(order, order + num_reqs, [&](int32_t a, int32_t b) { return m[a] > m[b]; });
    if (match_lens)
      for (int32_t r = 0; r < num_reqs; ++r) match_lens[r] = m[r];
    return PKV_OK;
  });
}

int32_t rt_serve_round(const rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                       const int32_t* after, const uint8_t* scheduled, int32_t window, int32_t order, int32_t batch,
                       int32_t* out_pick) {
  return guard([&]() -> int32_t {
    if (!t || num_reqs < 0 || window < 1 || batch < 1 || (order != RT_ORDER_FCFS && order != RT_ORDER_LPM) ||
        (num_reqs > 0 && (!tokens || !tok_indptr || !after || !scheduled || !out_pick)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_serve_round");
    // the waiting queue: the `window` oldest requests not yet scheduled; of those, the ones
    // whose predecessor was scheduled in an earlier round (or that have none)
    std::vector<int32_t> ready;
    int32_t waiting = 0;
    for (int32_t r = 0; r < num_reqs && waiting < window; ++r) {
      if (scheduled[r]) continue;
      ++waiting;
      const int32_t a = after[r];
      if (a >= r) return pkv::fail(PKV_ERR_INVAL, "request %d waits for request %d, which is not earlier", r, a);
      if (a < 0 || scheduled[a]) ready.push_back(r);
    }
    if (waiting == 0) return 0;
    if (ready.empty()) return pkv::fail(PKV_ERR_INVAL, "no waiting request is ready");
    if (order == RT_ORDER_LPM) {
      std::vector<int64_t> m(ready.size());
      for (size_t i = 0; i < ready.size(); ++i) {
        const int32_t r = ready[i];
        const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
        if (L < 0) return pkv::fail(PKV_ERR_INVAL, "request %d has a negative length", r);
        m[i] = t->peek(tokens + tok_indptr[r], L);
      }
      std::vector<size_t> idx(ready.size());
      for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
      std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) { return m[a] > m[b]; });
      std::vector<int32_t> sorted(ready.size());
      for (size_t i = 0; i < idx.size(); ++i) sorted[i] = ready[idx[i]];
      ready.swap(sorted);
    }
    const int32_t k = std::min<int32_t>(batch, (int32_t)ready.size());
    std::copy(ready.begin(), ready.begin() + k, out_pick);
    return k;
  });
}

int32_t rt_chunk_launch(const rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                        const int64_t* done, int32_t head, int64_t budget, int32_t* out_reqs, int64_t* out_ends) {
  return guard([&]() -> int32_t {
    if (!t || num_reqs < 0 || head < 0 || head > num_reqs || budget < 1 ||
        (num_reqs > 0 && (!tokens || !tok_indptr || !done || !out_reqs || !out_ends)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_chunk_launch");
    int64_t left = budget;
    int32_t k = 0;
    for (int32_t r = head; r < num_reqs && left > 0; ++r) {
      const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
      if (L < 0) return pkv::fail(PKV_ERR_INVAL, "request %d has a negative length", r);
      // a request already under way continues where its last chunk ended; a new one starts
      // after its cached prefix
      const int64_t start = done[r] >= 0 ? done[r] : t->peek(tokens + tok_indptr[r], L);
      if (start > L) return pkv::fail(PKV_ERR_INVAL, "request %d: %lld tokens done of %lld", r, (long long)start,
                                      (long long)L);
      const int64_t take = std::min(L - start, left);
      out_reqs[k] = r;
      out_ends[k] = start + take;
      ++k;
      left -= take;
    }
    return k;
  });
}

int64_t rt_dump_stats(const rt_tree* t, int64_t* out, int64_t cap) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  std::vector<int64_t> ids(t->live.begin(), t->live.end());
  std::sort(ids.begin(), ids.end());
  const int64_t need = 4 * (int64_t)ids.size();
  if (!out || cap < need) return need;
  int64_t k = 0;
  for (int64_t id : ids) {
    const Node& x = t->nodes[id];
    out[k++] = id;
    out[k++] = x.hits;
    out[k++] = x.created;
    out[k++] = x.priority;
  }
  return need;
}

int rt_inc_lock_ref(rt_tree* t, rt_node node) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  return t->inc_lock(node);
}

int rt_dec_lock_ref(rt_tree* t, rt_node node) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  return t->dec_lock(node);
}

int64_t rt_evict(rt_tree* t, int64_t num_tokens) {
  return guard([&]() -> int64_t {
    if (!t || num_tokens < 0) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_evict");
    return t->evict(num_tokens);
  });
}

int64_t rt_alloc(rt_tree* t, int64_t n, int32_t* out) {
  return guard([&]() -> int64_t {
    if (!t || (n > 0 && !out)) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_alloc");
    return t->alloc(n, out);
  });
}

int rt_free(rt_tree* t, const int32_t* slots, int64_t n) {
  if (!t || n < 0 || (n > 0 && !slots)) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_free");
  return t->free_slots(slots, n);
}

int rt_eviction_log_size(const rt_tree* t, int64_t* n_nodes, int64_t* n_slots) {
  if (!t || !n_nodes || !n_slots) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_eviction_log_size");
  *n_nodes = (int64_t)t->log_ids.size();
  *n_slots = (int64_t)t->log_slots.size();
  return PKV_OK;
}

int rt_set_eviction_log(rt_tree* t, int32_t enabled) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_set_eviction_log");
  t->log_on = enabled != 0;
  if (!t->log_on) {
    std::vector<int64_t>().swap(t->log_ids);
    std::vector<int64_t>().swap(t->log_lens);
    std::vector<int32_t>().swap(t->log_slots);
  }
  return PKV_OK;
}

int rt_take_eviction_log(rt_tree* t, int64_t* node_ids, int64_t* node_lens, int64_t nodes_cap, int32_t* slots,
                         int64_t slots_cap) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  const int64_t nn = (int64_t)t->log_ids.size(), ns = (int64_t)t->log_slots.size();
  if (nodes_cap < nn || slots_cap < ns || (nn && (!node_ids || !node_lens)) || (ns && !slots))
    return pkv::fail(PKV_ERR_INVAL, "eviction log needs %lld nodes / %lld slots", (long long)nn, (long long)ns);
  std::copy(t->log_ids.begin(), t->log_ids.end(), node_ids);
  std::copy(t->log_lens.begin(), t->log_lens.end(), node_lens);
  std::copy(t->log_slots.begin(), t->log_slots.end(), slots);
  t->log_ids.clear();
  t->log_lens.clear();
  t->log_slots.clear();
  return PKV_OK;
}

int64_t rt_evictable_size(const rt_tree* t) { return t ? t->evictable : PKV_ERR_INVAL; }
int64_t rt_protected_size(const rt_tree* t) { return t ? t->protected_ : PKV_ERR_INVAL; }
int64_t rt_free_size(const rt_tree* t) { return t ? t->count : PKV_ERR_INVAL; }
int64_t rt_clock(const rt_tree* t) { return t ? t->clock : PKV_ERR_INVAL; }

int64_t rt_copy_free_list(const rt_tree* t, int32_t* out, int64_t cap) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  if (cap >= t->count && out) {
    const int64_t R = (int64_t)t->ring.size();
    for (int64_t i = 0; i < t->count; ++i) out[i] = t->ring[(t->head + i) % R];
  }
  return t->count;
}

int64_t rt_dump(const rt_tree* t, int64_t* out, int64_t cap) {
  if (!t) return pkv::fail(PKV_ERR_INVAL, "tree is null");
  std::vector<int64_t> ids(t->live.begin(), t->live.end());
  std::sort(ids.begin(), ids.end());
  int64_t need = 0;
  for (int64_t id : ids) need += 5 + 2 * (int64_t)t->nodes[id].key.size();
  if (!out || cap < need) return need;
  int64_t k = 0;
  for (int64_t id : ids) {
    const Node& x = t->nodes[id];
    out[k++] = id;
    out[k++] = x.parent;
    out[k++] = x.lock_ref;
    out[k++] = x.last;
    out[k++] = (int64_t)x.key.size();
    for (int32_t v : x.key) out[k++] = v;
    for (int32_t v : x.value) out[k++] = v;
  }
  return need;
}

int64_t rt_prepare_extend(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                          int32_t* req_to_token, int64_t stride, int32_t* prefix_lens, int32_t* extend_lens,
                          int32_t* qo_indptr, int32_t* new_slots, int64_t new_cap, rt_node* out_last) {
  return rt_prepare_extend_prio(t, num_reqs, tokens, tok_indptr, nullptr, req_to_token, stride, prefix_lens,
                                extend_lens, qo_indptr, new_slots, new_cap, out_last);
}

int64_t rt_prepare_extend_prio(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                               const int32_t* priorities, int32_t* req_to_token, int64_t stride,
                               int32_t* prefix_lens, int32_t* extend_lens, int32_t* qo_indptr, int32_t* new_slots,
                               int64_t new_cap, rt_node* out_last) {
  return guard([&]() -> int64_t {
    if (!t || num_reqs < 0 || !tok_indptr || !req_to_token || !prefix_lens || !extend_lens || !qo_indptr ||
        !out_last || stride <= 0)
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_prepare_extend");
    int64_t total = 0;
    if (tok_indptr[0] != 0) return pkv::fail(PKV_ERR_INVAL, "tok_indptr[0] must be 0");
    for (int32_t r = 0; r < num_reqs; ++r) {
      int64_t L = tok_indptr[r + 1] - tok_indptr[r];
      if (L < 0 || L > stride || L > INT32_MAX)
        return pkv::fail(PKV_ERR_INVAL, "request %d has length %lld (stride %lld)", r, (long long)L,
                         (long long)stride);
      total += L;
    }
    if (total > 0 && (!tokens || !new_slots)) return pkv::fail(PKV_ERR_INVAL, "tokens/new_slots are null");
    if (new_cap < total)
      return pkv::fail(PKV_ERR_INVAL, "new_cap %lld < total tokens %lld", (long long)new_cap, (long long)total);
    for (int32_t r = 0; r < num_reqs; ++r) out_last[r] = -1;
    qo_indptr[0] = 0;
    int64_t n_new = 0;
    for (int32_t r = 0; r < num_reqs; ++r) {
      const int32_t* key = tokens + tok_indptr[r];
      const int64_t L = tok_indptr[r + 1] - tok_indptr[r];
      int32_t* row = req_to_token + (int64_t)r * stride;
      int64_t a = 0;
      const int64_t m = t->match(key, L, row, &a);
      t->inc_lock(a);
      int64_t rc = t->alloc(L - m, row + m);
      if (rc < 0) {
        t->dec_lock(a);
        return rc;
      }
      int64_t last = 0;
      const int64_t tm = t->insert_below(a, m, key, row, L, &last, priorities ? priorities[r] : 0);
      if (tm < 0) {
        t->dec_lock(a);
        return tm;
      }
      if (tm != m) {
        t->dec_lock(a);   // request r leaves no lock behind (its new tokens stay cached, unlocked)
        return pkv::fail(PKV_ERR_INTERNAL, "insert found %lld cached tokens after a match of %lld", (long long)tm,
                         (long long)m);
      }
      t->inc_lock(last);
      t->dec_lock(a);
      prefix_lens[r] = (int32_t)m;
      extend_lens[r] = (int32_t)(L - m);
      qo_indptr[r + 1] = (int32_t)(qo_indptr[r] + (L - m));
      std::memcpy(new_slots + n_new, row + m, sizeof(int32_t) * (L - m));
      n_new += L - m;
      out_last[r] = last;
    }
    return n_new;
  });
}

int rt_release(rt_tree* t, const rt_node* nodes, int32_t n) {
  if (!t || n < 0 || (n > 0 && !nodes)) return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_release");
  for (int32_t i = 0; i < n; ++i) {
    if (nodes[i] < 0) continue;
    int rc = t->dec_lock(nodes[i]);
    if (rc < 0) return rc;
  }
  return PKV_OK;
}

int32_t rt_chunk_prepare(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                         int64_t* done, rt_node* held, int32_t head, int64_t budget, int32_t* req_to_token,
                         int64_t stride, int32_t* prefix_lens, int32_t* extend_lens, int32_t* qo_indptr,
                         int32_t* new_slots, int64_t new_cap, int32_t* out_reqs, int64_t* out_ends,
                         int64_t* out_new) {
  return guard([&]() -> int32_t {
    if (!t || num_reqs < 0 || (num_reqs > 0 && (!done || !held || !out_new)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_chunk_prepare");
    const int32_t k = rt_chunk_launch(t, num_reqs, tokens, tok_indptr, done, head, budget, out_reqs, out_ends);
    if (k <= 0) {
      if (k == 0 && out_new) *out_new = 0;
      return k;
    }
    // the taken requests' truncated token lists, contiguous
    std::vector<int64_t> ip((size_t)k + 1, 0);
    for (int32_t i = 0; i < k; ++i) ip[(size_t)i + 1] = ip[(size_t)i] + out_ends[i];
    std::vector<int32_t> toks((size_t)ip[(size_t)k]);
    for (int32_t i = 0; i < k; ++i)
      std::copy(tokens + tok_indptr[out_reqs[i]], tokens + tok_indptr[out_reqs[i]] + out_ends[i],
                toks.begin() + ip[(size_t)i]);
    std::vector<rt_node> last((size_t)k, -1);
    const int64_t n_new = rt_prepare_extend(t, k, toks.data(), ip.data(), req_to_token, stride, prefix_lens,
                                            extend_lens, qo_indptr, new_slots, new_cap, last.data());
    if (n_new < 0) {
      rt_release(t, last.data(), k);   // the requests prepared before the failure
      return (int32_t)n_new;
    }
    // the previous chunk's lock is held until its continuation is prepared
    for (int32_t i = 0; i < k; ++i) {
      const int32_t r = out_reqs[i];
      if (held[r] >= 0) {
        const int rc = t->dec_lock(held[r]);
        if (rc < 0) return rc;
      }
      held[r] = last[(size_t)i];
      done[r] = out_ends[i];
    }
    *out_new = n_new;
    return k;
  });
}

int32_t rt_chunk_finish(rt_tree* t, int32_t num_reqs, const int64_t* tok_indptr, const int32_t* reqs, int32_t n,
                        const int64_t* done, rt_node* held, int32_t head) {
  return guard([&]() -> int32_t {
    if (!t || num_reqs < 0 || n < 0 || head < 0 || head > num_reqs ||
        (num_reqs > 0 && (!tok_indptr || !done || !held)) || (n > 0 && !reqs))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_chunk_finish");
    auto len = [&](int32_t r) { return tok_indptr[r + 1] - tok_indptr[r]; };
    for (int32_t i = 0; i < n; ++i) {
      const int32_t r = reqs[i];
      if (r < 0 || r >= num_reqs) return pkv::fail(PKV_ERR_INVAL, "request %d out of range", r);
      if (done[r] >= len(r) && held[r] >= 0) {
        const int rc = t->dec_lock(held[r]);
        if (rc < 0) return rc;
        held[r] = -1;
      }
    }
    while (head < num_reqs && done[head] >= len(head) && held[head] < 0) ++head;
    return head;
  });
}

int64_t rt_decode_step(rt_tree* t, int32_t batch, int32_t* req_to_token, int64_t stride, int32_t* seq_lens,
                       int32_t* out_slots) {
  return guard([&]() -> int64_t {
    if (!t || batch < 0 || (batch > 0 && (!req_to_token || !seq_lens || !out_slots)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_decode_step");
    for (int32_t b = 0; b < batch; ++b)
      if (seq_lens[b] < 0 || seq_lens[b] >= stride)
        return pkv::fail(PKV_ERR_INVAL, "sequence %d has length %d, stride %lld", b, seq_lens[b],
                         (long long)stride);
    int64_t rc = t->alloc(batch, out_slots);
    if (rc < 0) return rc;
    for (int32_t b = 0; b < batch; ++b) {
      req_to_token[(int64_t)b * stride + seq_lens[b]] = out_slots[b];
      ++seq_lens[b];
    }
    return batch;
  });
}

int rt_finish(rt_tree* t, int32_t n, const int32_t* tokens, const int64_t* tok_indptr, const int32_t* req_to_token,
              int64_t stride, const int32_t* prompt_lens, const rt_node* prompt_last, rt_node* out_end) {
  return guard([&]() -> int {
    if (!t || n < 0 || (n > 0 && (!tokens || !tok_indptr || !req_to_token || !prompt_lens || !prompt_last)))
      return pkv::fail(PKV_ERR_INVAL, "bad arguments to rt_finish");
    for (int32_t i = 0; i < n; ++i) {
      const int64_t L = tok_indptr[i + 1] - tok_indptr[i];
      if (L < 0 || L > stride || prompt_lens[i] < 0 || prompt_lens[i] > L)
        return pkv::fail(PKV_ERR_INVAL, "sequence %d: length %lld, prompt %d, stride %lld", i, (long long)L,
                         prompt_lens[i], (long long)stride);
      const int32_t* row = req_to_token + (int64_t)i * stride;
      int64_t end = 0;
      // resume below the prompt's end node when it still ends at the prompt (it is locked)
      const bool below = prompt_last[i] > 0 && t->is_live(prompt_last[i]) && t->depth(prompt_last[i]) == prompt_lens[i];
      int64_t m = below ? t->insert_below(prompt_last[i], prompt_lens[i], tokens + tok_indptr[i], row, L, &end)
                        : t->insert(tokens + tok_indptr[i], row, L, &end);
      if (m < 0) return (int)m;
      if (m > prompt_lens[i]) {
        int rc = t->free_slots(row + prompt_lens[i], m - prompt_lens[i]);
        if (rc < 0) return rc;
      }
      if (prompt_last[i] >= 0) {
        int rc = t->dec_lock(prompt_last[i]);
        if (rc < 0) return rc;
      }
      if (out_end) out_end[i] = end;
    }
    return PKV_OK;
  });
}

}  // extern "C"
