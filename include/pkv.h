/*
 * pkv.h - C ABI of libpkv.so: prefix-shared KV reuse for attention on MI355X (gfx950).
 *
 * Two halves:
 *   rt_*   a host radix tree over token ids whose values are KV slot indices of a
 *          token-granular KV pool, plus the pool's slot allocator.  Host memory only.
 *   pkv_*  HIP kernels that write new tokens' K/V into pool slots and run attention
 *          over K/V gathered through per-request slot rows.  Device memory only.
 *
 * Sources of the operations (the pages this library follows):
 *   [RC]  "[SGLang] RadixAttention: Radix Tree 기반 프리픽스 캐싱의 핵심" (radix-cache
 *         walkthrough): TreeNode fields, match_prefix with node split, _split_node,
 *         _insert_helper, the eviction heap, inc_lock_ref, and the worked example tree.
 *   [EX]  "論文解説: Efficiently Programming Large Language Models using SGLang"
 *         (RadixAttention explainer): the matched length is the longest common prefix;
 *         only the unmatched rest is prefilled; LRU eviction of unreferenced nodes.
 *   [OV]  "SGLang: Treating LLM Interactions as Programs ..." (overview): runtime flow
 *         "prefix match -> reuse / compute missing KV -> insert -> LRU evict", and the
 *         feedback of generated tokens into insertion.
 *   Attention is textbook scaled-dot-product attention (the pages do not state it):
 *   o_i = softmax(scale * q_i K[0..i]^T) V[0..i], query head h reads kv head
 *   h / (hq / hkv).
 *
 * Conventions
 *   - Every call returns >= 0 on success (0 or a count) and a negative PKV_ERR_* code on
 *     failure; nothing throws across the ABI.  pkv_last_error() returns a message for
 *     the calling thread's last failure (valid until that thread's next failing call).
 *   - rt_tree is not thread safe: one tree per thread, or external locking.
 *   - Slot ids are int32 in [0, num_slots).  Node ids are int64; 0 is the root; ids are
 *     never reused, so a stale id (an evicted node) is reported as PKV_ERR_NODE.
 *   - Ownership of slots: a slot is free (in the allocator), in flight (returned by
 *     rt_alloc, owned by the caller) or cached (held by a tree node).  rt_insert moves
 *     the in-flight slots of the newly inserted positions to cached; eviction moves
 *     cached slots back to free; rt_free moves in-flight slots back to free.
 *   - Kernel entry points take device pointers owned by the caller and enqueue work on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream); they return
 *     after enqueueing.  Buffers must stay alive until that work completes.  They never
 *     allocate device memory.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_ERR_INVAL (-1)       /* bad argument (null pointer, size, capacity)              */
#define PKV_ERR_OOM (-2)         /* not enough free slots even after evicting every unlocked leaf */
#define PKV_ERR_LOCK (-3)        /* unlock of a node whose lock reference is already 0       */
#define PKV_ERR_SLOT (-4)        /* slot out of range, or in the wrong ownership state       */
#define PKV_ERR_NODE (-5)        /* node id not live                                         */
#define PKV_ERR_HIP (-6)         /* a HIP runtime call failed                                */
#define PKV_ERR_UNSUPPORTED (-7) /* shape or dtype combination with no kernel                */
#define PKV_ERR_INTERNAL (-8)

typedef struct rt_tree rt_tree;
typedef int64_t rt_node;

const char* pkv_last_error(void);
int pkv_version(void);
/* Hash of the sources this library was built from (the binding refuses a stale build). */
const char* pkv_source_hash(void);

/* ----------------------------------------------------------------------------------
 * Radix tree and slot allocator (host)
 * -------------------------------------------------------------------------------- */

/* Create a tree over a pool of `num_slots` KV slots.  The allocator's free list is
 * `free_order[0..n_free)` (head first; distinct slots in range); NULL means
 * 0..num_slots-1 in order with n_free = num_slots.  Slots not listed are never handed
 * out.  The root node (id 0) carries lock reference 1 and is never evicted [RC figure
 * "Radix Tree 구조도"].  Logical clock starts at 0; node ids at 1. */
int rt_create(int64_t num_slots, const int32_t* free_order, int64_t n_free, rt_tree** out);
void rt_destroy(rt_tree* t);

/* Eviction policies [RC "Eviction 전략" (strategy selection) and the closing remarks on
 * several policies; RC "TreeNode 구조" for the hit count and priority fields].  Each is an
 * ascending heap key over unlocked leaves, ending in the node id:
 *   LRU (last access)              MRU (-last access)
 *   FIFO (creation clock)          FILO (-creation clock)
 *   LFU (hit count, last access)   PRIORITY (priority, last access)
 *   SLRU (hit count >= 2 ? 1 : 0, last access): a leaf hit at least twice sits in the
 *        protected segment and goes only after every probationary leaf.
 * Hit count = number of match calls that reused at least one token of the node (a split's
 * upper half starts from the old count and takes this match's hit; the lower half keeps
 * the old count).  Creation clock = clock of the insert that created the node (a split's
 * upper half inherits it).  Priority = max of the priorities of the inserts that walked
 * through or created the node (a split's upper half inherits it). */
typedef enum {
  RT_POLICY_LRU = 0, RT_POLICY_LFU = 1, RT_POLICY_SLRU = 2, RT_POLICY_FIFO = 3,
  RT_POLICY_MRU = 4, RT_POLICY_FILO = 5, RT_POLICY_PRIORITY = 6
} rt_policy;

/* rt_create with an eviction policy (rt_create is RT_POLICY_LRU).  An unknown policy
 * fails with PKV_ERR_INVAL. */
int rt_create_policy(int64_t num_slots, const int32_t* free_order, int64_t n_free, int32_t policy,
                     rt_tree** out);

/* Longest cached prefix of key[0..n) [RC "프리픽스 매칭: match_prefix"; EX matching formula].
 * Walks whole children keyed by their first token; if a child matches only partly
 * (including when the key ends inside it) the child is split at the match length
 * [RC "노드 분할"] and the walk stops.  Advances the logical clock by one and stamps
 * every visited node (and both halves of a split) with it.  Writes the matched slots
 * to out_slots (capacity n) and the id of the node ending the match to *out_last
 * (0 = root when nothing matched).  Returns the matched length. */
int64_t rt_match_prefix(rt_tree* t, const int32_t* key, int64_t n, int32_t* out_slots, rt_node* out_last);

/* Insert key -> slots [RC "삽입: _insert_helper"].  Walks and splits like match (clock
 * advanced by one, visited nodes stamped); the unmatched rest becomes a new leaf that
 * takes slots[m..n), which must be in flight; the new leaf's tokens count as evictable.
 * Returns the length m that was already cached; slots[0..m) are then duplicates that
 * stay owned by the caller (free them with rt_free).  *out_last = node ending the key. */
int64_t rt_insert(rt_tree* t, const int32_t* key, const int32_t* slots, int64_t n, rt_node* out_last);
/* rt_insert carrying a priority [RC "삽입: _insert_helper" priority argument]: every node the
 * walk passes (and a split's upper half) takes max(its priority, priority); a new leaf
 * takes priority.  rt_insert is priority 0.  Only RT_POLICY_PRIORITY reads it. */
int64_t rt_insert_priority(rt_tree* t, const int32_t* key, const int32_t* slots, int64_t n, int32_t priority,
                           rt_node* out_last);

/* Read-only prefix length: what rt_match_prefix would return for key[0..n), without a
 * split, a clock tick, a stamp or a hit.  Used to order waiting requests by cache hit
 * [OV and EX: cache-aware scheduling].  Returns the length or a negative error. */
int64_t rt_peek_prefix(const rt_tree* t, const int32_t* key, int64_t n);

/* Cache-aware order of waiting requests [OV and EX: longest-shared-prefix-first scheduling]:
 * order[0..num_reqs) = request indices sorted by descending rt_peek_prefix length, ties kept
 * in index (arrival) order; match_lens[r] (may be NULL) = request r's peek length.  The tree
 * is not changed.  Requests are tokens[tok_indptr[r] .. tok_indptr[r+1]). */
int rt_schedule_longest_prefix(const rt_tree* t, int32_t num_reqs, const int32_t* tokens,
                               const int64_t* tok_indptr, int32_t* order, int64_t* match_lens);

/* Lock references [RC "참조 카운트: lock_ref"]: +1 / -1 on every node from `node` up to,
 * not including, the root.  On 0 -> 1 a node's tokens move from the evictable to the
 * protected count (and back on 1 -> 0).  Locked nodes are never evicted.  Unlocking a
 * node whose count is 0 fails with PKV_ERR_LOCK and changes nothing. */
int rt_inc_lock_ref(rt_tree* t, rt_node node);
int rt_dec_lock_ref(rt_tree* t, rt_node node);

/* Evict at least num_tokens tokens [RC "Eviction 전략"; EX "LRU Evictionポリシー"]:
 * repeatedly remove the unlocked leaf with the smallest policy key (LRU: access time, node id), append
 * its slots to the free list's tail in key order, log it, and consider its parent once
 * the parent is an unlocked leaf.  Whole leaves only, so it may free more than asked.
 * Returns the number of tokens evicted (less than asked if nothing else is evictable). */
int64_t rt_evict(rt_tree* t, int64_t num_tokens);

/* Hand out n slots from the free list's head (first in, first out).  If fewer than n
 * are free it first evicts (n - free) tokens; if still short, returns PKV_ERR_OOM
 * (evictions already done stay done).  Slots become in flight.  Returns n.
 * [RC "Eviction 전략": eviction exists to give KV indices back to the pool's allocator
 * when new tokens need room; OV "Architectural Deep Dive" flowchart: compute the missing
 * KV, evicting least recently used entries under memory pressure.]  out: caller-owned host
 * array of n int32. */
int64_t rt_alloc(rt_tree* t, int64_t n, int32_t* out);

/* Return in-flight slots to the free list's tail, in the order given [RC "Eviction 전략":
 * freed KV indices go back to the pool allocator; "삽입: _insert_helper": the caller frees
 * the duplicate indices an insert reports].  A slot that is free already, cached by a node
 * or outside [0, num_slots) fails with PKV_ERR_SLOT and nothing is freed. */
int rt_free(rt_tree* t, const int32_t* slots, int64_t n);

/* Eviction log since the last take: node ids, their lengths, and the freed slots in
 * eviction order (the nodes [RC "Eviction 전략"] removes, one record per popped leaf).
 * rt_eviction_log_size reports the sizes; rt_take_eviction_log copies into caller-owned
 * host arrays and clears (PKV_ERR_INVAL, nothing cleared, if a capacity is too small). */
int rt_eviction_log_size(const rt_tree* t, int64_t* n_nodes, int64_t* n_slots);
int rt_take_eviction_log(rt_tree* t, int64_t* node_ids, int64_t* node_lens, int64_t nodes_cap,
                         int32_t* slots, int64_t slots_cap);

/* Turn the eviction log on (enabled != 0, the default for a new tree) or off.  A loop that
 * never takes the log should turn it off, or the log grows with every eviction.  Turning it
 * off also drops what it holds. */
int rt_set_eviction_log(rt_tree* t, int32_t enabled);

/* Token counters [RC "삽입: _insert_helper" (a new leaf's tokens count as evictable) and
 * "참조 카운트: lock_ref" (tokens move between evictable and protected on 0 <-> 1)]; the
 * free count is the allocator's [RC "Eviction 전략"].  PKV_ERR_INVAL for a null tree. */
int64_t rt_evictable_size(const rt_tree* t);   /* tokens in unlocked nodes  */
int64_t rt_protected_size(const rt_tree* t);   /* tokens in locked nodes    */
int64_t rt_free_size(const rt_tree* t);        /* slots on the free list    */
int64_t rt_clock(const rt_tree* t);
/* Copy the free list, head first, into out (capacity cap).  Returns its length. */
int64_t rt_copy_free_list(const rt_tree* t, int32_t* out, int64_t cap);
/* Serialise every live non-root node, by ascending id, as int64 records
 * [id, parent, lock_ref, last_access, len, key[len], slots[len]].  Returns the number
 * of int64 values; writes them only if cap is large enough. */
int64_t rt_dump(const rt_tree* t, int64_t* out, int64_t cap);
/* Per-node policy state of every live non-root node, by ascending id, as int64 records
 * [id, hit_count, creation_clock, priority].  Returns 4 x live nodes; writes only if cap
 * is large enough. */
int64_t rt_dump_stats(const rt_tree* t, int64_t* out, int64_t cap);

/* Batch driver: the hot path's host steps for one batch of requests, in order [OV
 * "Architectural Deep Dive" flowchart: prefix match, reuse the matched KV, compute the
 * missing KV, insert; RC "프리픽스 매칭", "참조 카운트", "삽입"; EX "プレフィックスマッチング
 * アルゴリズム": only the part after the matched prefix is prefilled].
 * For request r (tokens[tok_indptr[r] .. tok_indptr[r+1])), length L_r:
 *   match (split, stamp) -> lock the matched node -> allocate L_r - m_r slots (evicting
 *   on shortfall) -> insert (tokens, matched slots ++ new slots) -> lock the new end
 *   node, unlock the matched node.
 * Outputs (host arrays, caller-owned):
 *   req_to_token [num_reqs, stride]: row r = all L_r slots (entries past L_r untouched)
 *   prefix_lens[r] = m_r, extend_lens[r] = L_r - m_r, qo_indptr[0..num_reqs] = prefix
 *   sums of extend_lens (the rows of q / o / kv_scatter source for each request),
 *   new_slots[0..sum extend) = the fresh slots in the same row order,
 *   out_last[r] = node ending request r (locked until rt_release).
 * Requires stride >= max L_r and new_cap >= sum L_r.  On failure (e.g. PKV_ERR_OOM at
 * request r) requests before r stay prepared and locked, request r and later have
 * out_last = -1; release the prepared ones with rt_release.
 * Returns the total number of new tokens. */
int64_t rt_prepare_extend(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                          int32_t* req_to_token, int64_t stride, int32_t* prefix_lens,
                          int32_t* extend_lens, int32_t* qo_indptr, int32_t* new_slots, int64_t new_cap,
                          rt_node* out_last);
/* rt_prepare_extend whose insert of request r carries priorities[r] (NULL = all 0). */
int64_t rt_prepare_extend_prio(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                               const int32_t* priorities, int32_t* req_to_token, int64_t stride,
                               int32_t* prefix_lens, int32_t* extend_lens, int32_t* qo_indptr,
                               int32_t* new_slots, int64_t new_cap, rt_node* out_last);

/* Unlock out_last entries of a prepared batch (entries < 0 are skipped) once its kernels
 * have been enqueued [RC "참조 카운트: lock_ref": a request's nodes are protected from
 * eviction only while it uses them].  An entry already at lock 0 fails with PKV_ERR_LOCK
 * (the entries before it stay released). */
int rt_release(rt_tree* t, const rt_node* nodes, int32_t n);

/* One decode step for `batch` sequences [OV "Architectural Deep Dive": each generated
 * token gets KV of its own, which later feeds back into insertion]: allocate `batch` slots
 * in one call (evicting on shortfall, RC "Eviction 전략"); slot b is written to
 * req_to_token[b*stride + seq_lens[b]] and to out_slots[b], and seq_lens[b] is incremented.
 * Host arrays, caller-owned.  Requires seq_lens[b] < stride (else PKV_ERR_INVAL, nothing
 * allocated); PKV_ERR_OOM if the pool cannot supply `batch` slots. */
int64_t rt_decode_step(rt_tree* t, int32_t batch, int32_t* req_to_token, int64_t stride, int32_t* seq_lens,
                       int32_t* out_slots);

/* Finish sequences [OV feedback loop from generated tokens to insertion]: for each i,
 * insert (tokens_i, req_to_token row i [0..len_i)), free the caller's slots for
 * positions [prompt_lens[i], m) that the insert found already cached, and unlock
 * prompt_last[i].  out_end[i] = node ending the full sequence (may be NULL). */
int rt_finish(rt_tree* t, int32_t n, const int32_t* tokens, const int64_t* tok_indptr,
              const int32_t* req_to_token, int64_t stride, const int32_t* prompt_lens,
              const rt_node* prompt_last, rt_node* out_end);

/* One round of the serve loop [OV and EX: cache-aware scheduling, waiting requests served
 * longest cached prefix first rather than first come first served].  Requests
 * tokens[tok_indptr[r] .. tok_indptr[r+1]), r < num_reqs, arrive in index order; after[r] is
 * a request that must be scheduled in an earlier round (a conversation's previous turn), or
 * -1; scheduled[r] (0/1, host) marks those served in earlier rounds.  The waiting queue is
 * the `window` lowest-indexed requests not yet scheduled; the ready ones (after[r] < 0 or
 * scheduled[after[r]]) are taken in index order (order RT_ORDER_FCFS) or by descending
 * rt_peek_prefix length, ties in index order (RT_ORDER_LPM), and the first `batch` of them
 * are written to out_pick (caller-owned, capacity batch).  The tree is not changed (the
 * caller prepares, runs and releases the round, then marks its picks scheduled).  Returns
 * the number picked (0 once every request is scheduled); PKV_ERR_INVAL on bad arguments, an
 * after[r] not below r, or a queue with no ready request. */
#define RT_ORDER_FCFS 0
#define RT_ORDER_LPM 1
int32_t rt_serve_round(const rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                       const int32_t* after, const uint8_t* scheduled, int32_t window, int32_t order, int32_t batch,
                       int32_t* out_pick);

/* One launch of chunked prefill (a cap of `budget` new tokens per extend launch) [the
 * deployment-tuning page's chunked-prefill option; requests keep their order]: from request
 * `head` on, each request contributes min(its tokens not yet prefilled, budget left) and the
 * walk stops when the budget is spent, so only the last request taken may be cut.  A
 * request's tokens not yet prefilled start at done[r] when done[r] >= 0 (it is under way:
 * its earlier chunks are cached and locked) and otherwise after its cached prefix
 * (rt_peek_prefix, read-only).  Writes the requests taken to out_reqs and the end position of
 * each one's chunk to out_ends (caller-owned, capacity num_reqs - head); the caller prepares
 * the launch as the truncated token lists [0, end).  Returns the number taken;
 * PKV_ERR_INVAL on bad arguments. */
int32_t rt_chunk_launch(const rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                        const int64_t* done, int32_t head, int64_t budget, int32_t* out_reqs, int64_t* out_ends);

/* One launch of chunked prefill from cut to host tables [the deployment-tuning page's
 * chunked-prefill option; the radix tree's prefix match lets a request's next chunk reuse its
 * earlier ones: RC "프리픽스 매칭"]: the requests rt_chunk_launch takes from `head` (at most
 * `budget` new tokens), prepared with rt_prepare_extend as their truncated token lists
 * [0, end_r), in order; then for each taken request r the end node of its previous chunk
 * (held[r] >= 0) is unlocked and held[r] = the new chunk's end node, done[r] = end_r.
 * done and held [num_reqs] are caller-owned state carried across launches, both -1 before
 * the first.  Outputs: out_reqs / out_ends (capacity num_reqs - head), the extend tables as
 * rt_prepare_extend writes them for the taken requests in order (new_cap >= the sum of their
 * ends), *out_new = the new tokens.  Returns the number of requests taken (0 when none is
 * left); a negative error (a failed prepare leaves done / held unchanged and unlocks what it
 * prepared). */
int32_t rt_chunk_prepare(rt_tree* t, int32_t num_reqs, const int32_t* tokens, const int64_t* tok_indptr,
                         int64_t* done, rt_node* held, int32_t head, int64_t budget, int32_t* req_to_token,
                         int64_t stride, int32_t* prefix_lens, int32_t* extend_lens, int32_t* qo_indptr,
                         int32_t* new_slots, int64_t new_cap, int32_t* out_reqs, int64_t* out_ends,
                         int64_t* out_new);
/* After a chunked-prefill launch's kernels: the taken requests reqs[0..n) that reached their
 * end (done[r] >= their length) have their end node unlocked and held[r] = -1.  Returns the
 * new head: the first request from `head` on that is not finished (num_reqs when all are). */
int32_t rt_chunk_finish(rt_tree* t, int32_t num_reqs, const int64_t* tok_indptr, const int32_t* reqs, int32_t n,
                        const int64_t* done, rt_node* held, int32_t head);

/* ----------------------------------------------------------------------------------
 * Kernels (device)
 * -------------------------------------------------------------------------------- */

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Write new tokens' K/V into their pool slots [RC "핵심 자료구조: TreeNode": a node's value
 * holds one KV-pool index per token; OV flowchart: the missing KV is computed and stored]:
 *   k_pool[slots[i], h, :] = cvt(k_src[i, h, :]),  same for V,  i < n, h < hkv.
 * Layouts: k_src/v_src [n, hkv, d] row-major in src_dtype; pools [num_slots, hkv, d]
 * row-major in pool_dtype; slots device int32 [n].
 * Supported: (F32 -> F32), (BF16 -> BF16) copies, and (BF16 -> FP8_E4M3) quantisation
 * code = round-to-nearest-even(float32(x * inv_scale[h])) saturated to +-448 (OCP
 * E4M3, sign kept), with k_inv_scale/v_inv_scale device float32 [hkv].
 * Slots must be distinct (duplicates race); a slot outside [0, num_slots) is skipped (its
 * token is not written; a PKV_DEBUG build rejects such a list, and repeated slots, with
 * PKV_ERR_SLOT before launching).  d in {64, 128}. */
int pkv_kv_scatter(const void* k_src, const void* v_src, int32_t src_dtype, const int32_t* slots, int64_t n,
                   void* k_pool, void* v_pool, int32_t pool_dtype, int64_t num_slots, int32_t hkv, int32_t d,
                   const float* k_inv_scale, const float* v_inv_scale, void* stream);

/* Device side of one decode step's table emit (rt_decode_step fills the host table):
 * req_to_token[b*stride + seq_lens[b] - 1] = slots[b] for b < batch, where seq_lens are the
 * lengths AFTER the step (the new token included).  Entries whose position falls outside
 * [0, stride) are skipped.  All pointers are device pointers. */
int pkv_append_slots(int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, const int32_t* slots,
                     int32_t batch, void* stream);

/* Host-side plan for pkv_extend_attention: split each request's extend rows into query
 * tiles of `tile` tokens and order the tiles by descending work (context length), so
 * the longest tiles start first.  prefix_lens/extend_lens are HOST arrays [num_reqs].
 * Writes work items (request, first extend row of the tile) as int32 pairs to
 * out_work[2*i], out_work[2*i+1]; returns the number of items (PKV_ERR_INVAL if
 * work_cap is too small; pkv_extend_plan_size gives the exact count). */
int64_t pkv_extend_plan_size(const int32_t* extend_lens, int32_t num_reqs, int32_t tile);
int64_t pkv_extend_plan(const int32_t* prefix_lens, const int32_t* extend_lens, int32_t num_reqs, int32_t tile,
                        int32_t* out_work, int64_t work_cap);
/* Query-tile size (in tokens) pkv_extend_attention expects for a shape. */
int32_t pkv_extend_tile(int32_t qo_dtype, int32_t pool_dtype, int32_t hq, int32_t hkv, int32_t d);

/* Extend (prefill of the unmatched suffix over a reused prefix) [EX: only the part
 * after the matched prefix is computed].  For request r with prefix p = prefix_lens[r]
 * and e = extend_lens[r] rows starting at q row qo_indptr[r], extend row j (token
 * position i = p + j), query head h, kv head g = h / (hq / hkv):
 *   o[qo_indptr[r]+j, h, :] = softmax_k(sm_scale * <q[.., h, :], K[k, g, :]>) V[k, g, :]
 *   over k = 0..i, with K[k] = k_pool[req_to_token[r*stride + k]] (full over the
 *   prefix, causal over the suffix).
 * Layouts: q, o [total_q, hq, d] in qo_dtype (F32 or BF16); pools [num_slots, hkv, d];
 * req_to_token device int32 [num_reqs, stride]; prefix_lens, extend_lens, qo_indptr
 * device int32; work device int32 [n_work, 2] from pkv_extend_plan with the tile of
 * pkv_extend_tile.  fp8 pools: the dequantised value is code * k_scale[g] (v_scale[g]),
 * device float32 [hkv]; the scale is folded into the float32 logits / output.
 * Supported: (F32 q/o, F32 pool, d 64 or 128) and (BF16 q/o, BF16 or FP8_E4M3 pool, d 64)
 * for any hq % hkv == 0 (VALU kernel); (BF16 q/o, BF16 or FP8_E4M3 pool, d 128) with hq / hkv
 * in {1, 2, 4, 8} and a slot of at most 16,383 bytes (MFMA kernels).  Softmax and
 * accumulation in float32. */
int pkv_extend_attention(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                         int32_t pool_dtype, int64_t num_slots, const float* k_scale, const float* v_scale,
                         const int32_t* req_to_token, int64_t stride, const int32_t* prefix_lens,
                         const int32_t* extend_lens, const int32_t* qo_indptr, int32_t num_reqs,
                         const int32_t* work, int64_t n_work, int32_t hq, int32_t hkv, int32_t d,
                         float sm_scale, void* stream);

/* Decode [OV "Architectural Deep Dive": the generation step; EX: the matched prefix's KV is
 * reused, not recomputed]: one query token per sequence, the newest one (position
 * seq_lens[b] - 1, its own K/V included), over its whole cached context (textbook scaled
 * dot-product attention; the pages do not state the formula).  Split-K: the context is cut into chunks of `chunk` tokens; one
 * partial (running max, running sum, unnormalised output) per (sequence, q head, chunk)
 * goes to the workspace, then a reduce merges the chunks by log-sum-exp:
 *   M = max_s m_s,  o = sum_s exp(m_s - M) acc_s / sum_s exp(m_s - M) l_s.
 * Layouts: q, o [batch, hq, d] in qo_dtype; req_to_token device int32 [batch, stride];
 * seq_lens device int32 [batch], each in [1, max_seq_len].  chunk: tokens per split, a
 * multiple of 64, or 0 for automatic.  workspace: device memory of at least
 * pkv_decode_workspace_bytes(batch, hq, d, max_seq_len, chunk) bytes.
 * Supported: (F32 q/o, F32 pool) and (BF16 q/o, BF16 or FP8_E4M3 pool), d 64 or 128, with
 * hq / hkv in {1, 2, 4, 8}.  Slots past the pool read the pool's last
 * slot (no access leaves the pools).  Errors: PKV_ERR_INVAL (sizes, null pointers, a
 * workspace too small), PKV_ERR_UNSUPPORTED (shape), PKV_ERR_HIP (launch).
 * pkv_decode_workspace_bytes: the caller-owned device workspace the split phase needs for
 * this decode (one partial per (sequence, q head, chunk): running max, running sum and d
 * output values, float32); 0 for bad sizes. */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t d, int32_t max_seq_len, int32_t chunk);
/* The automatic chunk: 1024 tokens, halved (not below 128) while the split phase would launch
 * fewer than 2048 workgroups (one per (sequence, chunk) when hkv is 2, 4 or 8, one per
 * (sequence, chunk, group of 8 kv heads) for other multiples of 8, one per (sequence, chunk,
 * kv head) otherwise). */
int32_t pkv_decode_chunk(int32_t batch, int32_t hkv, int32_t max_seq_len);
int pkv_decode_attention(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                         int32_t pool_dtype, int64_t num_slots, const float* k_scale, const float* v_scale,
                         const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                         int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t chunk,
                         void* workspace, size_t ws_bytes, void* stream);

/* Shared-prefix decode.  The radix tree gives every request that matches a cached prefix the
 * slots of that prefix [RadixAttention: prefix matching and KV cache reuse], so the decode
 * sequences of a batch that share a prefix hold its K/V rows in the same slots.  A chunk of
 * such rows can be read once for all of them: their newest tokens are stacked as the query
 * rows of one MFMA tile (up to pkv_decode_shared_rows rows per kv head) and the chunk's split
 * partial is written for every one of them; the split phase then skips those chunks.
 *
 * pkv_decode_shared_plan (host): from the HOST slot rows req_to_token [batch, stride] and
 * seq_lens [batch] (each in [1, stride]), partition the sequences chunk by chunk: at chunk k
 * the sequences of a group (all equal on chunks 0..k-1) whose chunk k (whole, inside their
 * context) is slot for slot equal form a job (members, k), which is partitioned again at
 * k + 1; a sequence left alone stops sharing at k.  The jobs of one member set at
 * consecutive chunks are merged into spans of at most max_span chunks (one workgroup then
 * reads the whole span and writes one partial).  Outputs (caller-owned host arrays):
 *   members [batch]  sequence indices, each job's members contiguous;
 *   skip [batch]     chunks 0..skip[b]-1 of sequence b are covered by jobs;
 *   items [cap, 4]   (index of the first member in `members`, member count <= rows, first
 *                    chunk, span in chunks), a span cut into items of at most `rows` members.
 * chunk: the split chunk the decode will use (a multiple of 64).  rows_from_tree = 1 when
 * the rows come from one radix tree (as rt_prepare_extend / rt_decode_step write them, while
 * the batch holds its locks): a slot then belongs to one node at one depth, so rows that hold
 * the same slot at a position agree on every earlier position and only each chunk's last
 * slot is compared; 0 compares every slot.  private_items = 1 appends, after the shared
 * items, one-member items (spans of at most max_span chunks) over each sequence's remaining
 * chunks up to the one holding its newest token, and sets skip[b] = ceil(seq_lens[b] / chunk):
 * the shared-prefix kernel then takes the whole step (the kernel masks positions past each
 * member's newest token), which pays when those tails are few and short.  Returns the number
 * of items, PKV_ERR_INVAL on bad sizes or when items_cap is too small (the message gives the
 * count).  The plan stays valid while the sequences only grow (new tokens are private; a
 * sequence that grows into a chunk past skip[b] has it done by the split phase). */
int64_t pkv_decode_shared_plan(const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                               int32_t chunk, int32_t rows, int32_t max_span, int32_t rows_from_tree,
                               int32_t private_items, int32_t* members, int32_t* skip, int32_t* items,
                               int64_t items_cap);
/* Query rows (member sequences) per shared-prefix item for a shape: 128 / (hq / hkv), or
 * PKV_ERR_UNSUPPORTED (shared-prefix decode needs BF16 q/o, a BF16 or FP8_E4M3 pool, d = 128,
 * hq / hkv in {1, 2, 4, 8}). */
int32_t pkv_decode_shared_rows(int32_t qo_dtype, int32_t pool_dtype, int32_t hq, int32_t hkv, int32_t d);
/* pkv_decode_attention with a shared-prefix plan: members, skip, items are DEVICE copies of
 * pkv_decode_shared_plan's outputs (n_items of them) for the same slot rows and the same
 * (nonzero) chunk; first_split: the smallest skip[b] over the sequences whose context reaches
 * past chunk skip[b] (0 is always correct); the split phase launches chunks first_split and
 * later only, and not at all when first_split >= ceil(max_seq_len / chunk).  Items whose
 * members or chunk fall outside the batch or the workspace are
 * ignored (their partials are then left unwritten, so the result is wrong but no access
 * leaves the buffers).  Same result as pkv_decode_attention up to float32 summation order;
 * n_items = 0 is pkv_decode_attention. */
int pkv_decode_attention_shared(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                                int32_t pool_dtype, int64_t num_slots, const float* k_scale, const float* v_scale,
                                const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t chunk,
                                const int32_t* members, const int32_t* skip, const int32_t* items, int64_t n_items,
                                int32_t first_split, void* workspace, size_t ws_bytes, void* stream);

/* Decode for callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pkv_decode_attention_shared (n_items = 0 is
 * the plain decode) with the split partials in a file-scope device array of
 * PKV_DECODE_STATIC_SCRATCH_BYTES instead of a caller workspace.  Each GPU the library runs on
 * holds its own copy of the array until the process ends; its address is looked up once per
 * device on the first call there.  Calls that overlap on one GPU share the array and race.
 * chunk = 0 takes the automatic chunk, doubled while the partials do not fit when there is no
 * plan (n_items = 0 and first_split = 0; a plan is tied to the chunk it was made for); a call whose
 * partials still exceed the array (at the chunk given) fails with PKV_ERR_INVAL and a message
 * giving the sizes.  Allocates nothing; other arguments and errors as for
 * pkv_decode_attention_shared. */
#define PKV_DECODE_STATIC_SCRATCH_BYTES (64LL << 20)
int pkv_decode_attention_static(const void* q, void* o, int32_t qo_dtype, const void* k_pool, const void* v_pool,
                                int32_t pool_dtype, int64_t num_slots, const float* k_scale, const float* v_scale,
                                const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                                int32_t max_seq_len, int32_t hq, int32_t hkv, int32_t d, float sm_scale, int32_t chunk,
                                const int32_t* members, const int32_t* skip, const int32_t* items, int64_t n_items,
                                int32_t first_split, void* stream);

/* first_split value meaning "no split phase at all". */
#define PKV_NO_SPLIT_PHASE (1 << 30)
/* The first chunk the split phase must launch for a plan's skip [batch] at the current
 * lengths seq_lens [batch] (host arrays): the smallest skip[b] over the sequences whose
 * context holds a chunk at or past skip[b], or PKV_NO_SPLIT_PHASE when the plan's items
 * cover every context.  A plan made at one step stays valid while the sequences grow; this
 * is recomputed at each step from that step's lengths.  PKV_ERR_INVAL on bad arguments. */
int32_t pkv_decode_first_split(const int32_t* skip, const int32_t* seq_lens, int32_t batch, int32_t chunk);
/* Item capacity pkv_decode_plan (and pkv_decode_shared_plan with any max_span and
 * private_items) may need for these lengths, stride, chunk and rows per item. */
int64_t pkv_decode_plan_items_cap(const int32_t* seq_lens, int32_t batch, int64_t stride, int32_t chunk, int32_t rows);
/* The shared-prefix plan with its choices made [the radix tree gives sequences that share a
 * prefix the same slots: RC "프리픽스 매칭"; EX: matched KV is reused]: pkv_decode_shared_plan
 * over rows from one radix tree.  When the shared items and the private tails together need
 * at most private_max_workgroups workgroups (items x hkv), the tails become one-member items
 * too.  Items then span the number of chunks `span` in 1 .. min(longest context in chunks,
 * 64) that minimizes ceil(items(span) x hkv / resident_workgroups) x (4 + span x chunk / 64)
 * (launch rounds of resident_workgroups, each as long as its longest item: 4 tiles of fixed
 * cost plus its tiles), the longer span on a tie.  Outputs as for pkv_decode_shared_plan,
 * plus *first_split = pkv_decode_first_split at these lengths.  Returns the number of items
 * (0: nothing is shared, decode without a plan; *first_split 0); PKV_ERR_INVAL on bad
 * arguments. */
int64_t pkv_decode_plan(const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                        int32_t chunk, int32_t rows, int32_t hkv, int32_t resident_workgroups,
                        int32_t private_max_workgroups, int32_t* members, int32_t* skip, int32_t* items,
                        int64_t items_cap, int32_t* first_split);

/* ----------------------------------------------------------------------------------
 * Measurement helper (device)
 * -------------------------------------------------------------------------------- */

/* A plain streaming read of `bytes` (a positive multiple of 16) of device memory at `buf`:
 * the rate a read-only kernel reaches on this GPU's HBM, set beside the published peak when
 * the HBM-bound kernels are measured.  `out` is caller-owned device memory of
 * pkv_stream_read_words() uint32 words (written so the loads stay live; the values mean
 * nothing).  Enqueued on `stream`; PKV_ERR_INVAL on bad arguments. */
int32_t pkv_stream_read_words(void);
int pkv_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
