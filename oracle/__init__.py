"""Oracle: a plain, slow, obviously correct CPU statement of the prefix-shared KV path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
CPU-baseline leg may import anything from this package; the product path
(the C-ABI library and its Python binding) never does, and shares no code with
it.  Inputs come from the ``workloads`` package (seeded draws, no method
arithmetic).

Contents
- ``radix_tree``: the radix tree over token ids with token-granular KV slots
  (prefix match with node split, insert, lock references, LRU leaf eviction)
  and the slot free list, after the radix-cache walkthrough page
  ("[SGLang] RadixAttention: Radix Tree 기반 프리픽스 캐싱의 핵심",
  sections "프리픽스 매칭", "노드 분할", "삽입", "Eviction 전략", "참조 카운트").
- ``driver``: the sequential per-request driver that turns a batch into a
  ``req_to_token`` table (match, lock, allocate, insert, relock) and the
  decode-step and finish steps.
- ``attention``: float64 scaled-dot-product attention recomputed from each
  request's full token sequence (no tree, no slots).
- ``fp8``: the OCP FP8 E4M3 code table, round-to-nearest-even saturating
  encoder and decoder.

Every function is pinned by the ``-m "not gpu"`` tests (worked example of the
radix-cache page, split picture, brute-force longest-common-prefix model,
lock/evict invariants, closed forms, PyTorch float64 attention, OCP code
table).  No function here is "parity unpinned".
"""
