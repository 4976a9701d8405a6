// Host-side plan of the shared-prefix decode: which leading context chunks several sequences
// of a decode batch hold in the same pool slots.
//
// The radix tree hands every request that matches a cached prefix the slots of that prefix
// (RadixAttention, "prefix matching" / "KV cache reuse"): sequences that share a prefix
// share its K/V rows in the pool, slot for slot.  Their decode steps then read the same
// rows; a chunk of such rows can be streamed once for all of them, with the query rows of
// every sharing sequence stacked into one dense product (a multi-query tile).
//
// The plan is computed from the slot rows alone.  Sequences are partitioned chunk by chunk:
// at level k the members of a group (which all agree on chunks 0 .. k-1) are sorted by the
// first slot of chunk k, and members whose whole chunk k equals that of the first member of
// their run form a sub-group.  A sub-group of two or more sequences is a job (members,
// chunk k) and is partitioned again at level k + 1; a sequence left alone stops sharing at
// chunk k.  Only whole chunks inside a sequence's context take part.  The jobs of one member
// set at consecutive levels (a group that does not split) are merged into spans of up to
// max_span chunks, so a long shared prefix is read by fewer, longer workgroups that write one
// partial per span instead of one per chunk; spans are cut into items of at most `rows`
// members, the query rows one kernel workgroup holds per kv head.
//
// With private_items, every sequence's remaining chunks (from skip[b] to the chunk holding
// its newest token) become one-member items too, spans of up to max_span chunks, and skip[b]
// moves past them: the MFMA kernel then takes the whole step and the split phase has nothing
// left (worth it when those tails are short and few, where the split phase's workgroups are
// latency-bound; the kernel masks the positions past each member's newest token).
//
// Rows that come from one radix tree need no whole-chunk comparison: a slot belongs to one
// node at one depth, so two rows holding the same slot at a position hold the same slots at
// every earlier position too, and comparing a chunk's last slot decides the whole chunk.
// With rows_from_tree = 0 every chunk is compared slot for slot.

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "common.h"

using namespace pkv;

extern "C" int64_t pkv_decode_shared_plan(const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens,
                                          int32_t batch, int32_t chunk, int32_t rows, int32_t max_span,
                                          int32_t rows_from_tree, int32_t private_items, int32_t* members,
                                          int32_t* skip, int32_t* items, int64_t items_cap) {
  if (batch < 0 || stride <= 0 || chunk < 64 || chunk % 64 || rows <= 0 || max_span <= 0 || items_cap < 0)
    return fail(PKV_ERR_INVAL, "decode plan: bad sizes (batch %d stride %lld chunk %d rows %d span %d)", batch,
                (long long)stride, chunk, rows, max_span);
  if (batch == 0) return 0;
  if (!req_to_token || !seq_lens || !members || !skip || (items_cap > 0 && !items))
    return fail(PKV_ERR_INVAL, "decode plan: null pointer");
  std::vector<int32_t> full((size_t)batch);   // whole chunks inside each context
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 1 || L > stride) return fail(PKV_ERR_INVAL, "decode plan: seq_lens[%d] = %lld", b, (long long)L);
    full[b] = (int32_t)(L / chunk);
    members[b] = b;
    skip[b] = 0;
  }
  const size_t chunk_bytes = (size_t)chunk * sizeof(int32_t);
  auto row = [&](int32_t b, int32_t k) { return req_to_token + (int64_t)b * stride + (int64_t)k * chunk; };
  struct Job {
    int32_t lo, cnt, k;   // members[lo, lo + cnt) share chunk k
  };
  std::vector<Job> jobs;
  struct Range {
    int32_t lo, hi, k;   // members[lo, hi) agree on chunks 0 .. k-1
  };
  std::vector<Range> todo{Range{0, batch, 0}};
  while (!todo.empty()) {
    const Range r = todo.back();
    todo.pop_back();
    int32_t* m = members + r.lo;
    const int32_t n = r.hi - r.lo;
    // members whose context holds chunk k first, ordered by the chunk's first slot (then by
    // sequence, so the plan is deterministic); the others stop sharing here
    int32_t* mid = std::stable_partition(m, m + n, [&](int32_t b) { return full[b] > r.k; });
    for (int32_t* p = mid; p < m + n; ++p) skip[*p] = r.k;
    std::stable_sort(m, mid, [&](int32_t a, int32_t b) {
      const int32_t sa = row(a, r.k)[0], sb = row(b, r.k)[0];
      return sa != sb ? sa < sb : a < b;
    });
    // runs of equal first slot, each split into the members equal to the run's first one
    // over the whole chunk (moved to the front) and the rest, which stop sharing here
    std::vector<Range> next;
    for (int32_t* a = m; a < mid;) {
      int32_t* e = a + 1;
      while (e < mid && row(*e, r.k)[0] == row(*a, r.k)[0]) ++e;
      const int32_t* ref = row(*a, r.k);
      int32_t* same_end = std::stable_partition(a + 1, e, [&](int32_t b) {
        return rows_from_tree ? row(b, r.k)[chunk - 1] == ref[chunk - 1]
                              : std::memcmp(row(b, r.k), ref, chunk_bytes) == 0;
      });
      for (int32_t* p = same_end; p < e; ++p) skip[*p] = r.k;
      const int32_t cnt = (int32_t)(same_end - a);
      if (cnt >= 2) {
        const int32_t lo = (int32_t)(a - members);
        jobs.push_back(Job{lo, cnt, r.k});
        next.push_back(Range{lo, lo + cnt, r.k + 1});
      } else {
        skip[*a] = r.k;
      }
      a = e;
    }
    // depth first, lowest members first
    for (auto it = next.rbegin(); it != next.rend(); ++it) todo.push_back(*it);
  }
  // spans: the jobs of one member set (same range of `members`) at consecutive chunks, up to
  // max_span chunks each, in order of first chunk; then items of at most `rows` members
  std::stable_sort(jobs.begin(), jobs.end(), [](const Job& x, const Job& y) {
    return x.lo != y.lo ? x.lo < y.lo : (x.cnt != y.cnt ? x.cnt > y.cnt : x.k < y.k);
  });
  struct Span {
    int32_t lo, cnt, k, span;
  };
  std::vector<Span> spans;
  for (const Job& j : jobs) {
    if (!spans.empty()) {
      Span& last = spans.back();
      if (last.lo == j.lo && last.cnt == j.cnt && last.k + last.span == j.k && last.span < max_span) {
        ++last.span;
        continue;
      }
    }
    spans.push_back(Span{j.lo, j.cnt, j.k, 1});
  }
  std::stable_sort(spans.begin(), spans.end(),
                   [](const Span& x, const Span& y) { return x.k != y.k ? x.k < y.k : x.lo < y.lo; });
  int64_t n_items = 0;
  auto emit = [&](int32_t m0, int32_t nm, int32_t k, int32_t span) {
    if (n_items < items_cap) {
      int32_t* it = items + 4 * n_items;
      it[0] = m0;
      it[1] = nm;
      it[2] = k;
      it[3] = span;
    }
    ++n_items;
  };
  for (const Span& sp : spans)
    for (int32_t i = 0; i < sp.cnt; i += rows) emit(sp.lo + i, std::min(rows, sp.cnt - i), sp.k, sp.span);
  if (private_items) {
    for (int32_t i = 0; i < batch; ++i) {
      const int32_t b = members[i];
      const int32_t last = (int32_t)((seq_lens[b] - 1) / chunk);   // the chunk of the newest token
      for (int32_t k = skip[b]; k <= last; k += max_span) emit(i, 1, k, std::min(max_span, last - k + 1));
      skip[b] = last + 1;
    }
  }
  if (n_items > items_cap) return fail(PKV_ERR_INVAL, "decode plan: needs %lld items", (long long)n_items);
  return n_items;
}

extern "C" int32_t pkv_decode_first_split(const int32_t* skip, const int32_t* seq_lens, int32_t batch, int32_t chunk) {
  if (batch < 0 || chunk <= 0 || (batch > 0 && (!skip || !seq_lens)))
    return fail(PKV_ERR_INVAL, "first split: bad arguments (batch %d chunk %d)", batch, chunk);
  int32_t first = PKV_NO_SPLIT_PHASE;
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_lens[b] < 1 || skip[b] < 0) return fail(PKV_ERR_INVAL, "first split: sequence %d", b);
    const int64_t chunks = ((int64_t)seq_lens[b] + chunk - 1) / chunk;   // chunks holding its context
    if (chunks > skip[b]) first = std::min(first, skip[b]);
  }
  return first;
}

extern "C" int64_t pkv_decode_plan_items_cap(const int32_t* seq_lens, int32_t batch, int64_t stride, int32_t chunk,
                                             int32_t rows) {
  if (batch < 0 || stride <= 0 || chunk <= 0 || rows <= 0 || (batch > 0 && !seq_lens))
    return fail(PKV_ERR_INVAL, "decode plan capacity: bad arguments");
  // a job holds two members or more, so a chunk level makes at most batch / 2 items when an
  // item takes two rows or more (one per member with one row per item); private items add at
  // most one per chunk of each context
  int64_t cap = (int64_t)batch * (stride / chunk) / (rows >= 2 ? 2 : 1) + 1;
  for (int32_t b = 0; b < batch; ++b) cap += ((int64_t)seq_lens[b] + chunk - 1) / chunk;
  return cap;
}

extern "C" int64_t pkv_decode_plan(const int32_t* req_to_token, int64_t stride, const int32_t* seq_lens, int32_t batch,
                                   int32_t chunk, int32_t rows, int32_t hkv, int32_t resident_workgroups,
                                   int32_t private_max_workgroups, int32_t* members, int32_t* skip, int32_t* items,
                                   int64_t items_cap, int32_t* first_split) {
  if (hkv <= 0 || resident_workgroups <= 0 || chunk <= 0 || !first_split)
    return fail(PKV_ERR_INVAL, "decode plan: bad arguments (hkv %d, resident_workgroups %d, chunk %d)", hkv,
                resident_workgroups, chunk);
  *first_split = 0;
  // rows from one radix tree (the caller holds the batch's locks): each chunk's last slot decides
  int64_t n = pkv_decode_shared_plan(req_to_token, stride, seq_lens, batch, chunk, rows, 1, 1, 0, members, skip,
                                     items, items_cap);
  if (n <= 0) return n;
  int64_t tails = 0;   // private chunks left to the split phase
  int64_t longest = 1;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t c = ((int64_t)seq_lens[b] + chunk - 1) / chunk;
    tails += c - skip[b];
    longest = std::max(longest, c);
  }
  // few, short private tails: one-member items take them too, and the split phase (whose
  // workgroups would be latency-bound) is not launched
  const bool priv = (n + tails) * hkv <= (int64_t)private_max_workgroups;
  // Span: workgroups start in rounds of about resident_workgroups (what the GPU holds at
  // once) and a round lasts about as long as its longest item, so a plan costs about
  //   ceil(items x hkv / resident_workgroups) x (kItemFixed + span x chunk / 64)  tile times,
  // kItemFixed being a workgroup's fixed cost in tiles (its q rows, the pipeline fill, the
  // partial store).  The cheapest span in 1 .. min(longest context in chunks, 64) is taken,
  // the longer one on a tie (fewer partials to write and merge).
  constexpr int64_t kItemFixed = 4;
  const int64_t tiles_per_chunk = std::max<int64_t>(chunk / 64, 1);
  const int32_t max_span = (int32_t)std::min<int64_t>(longest, 64);
  int32_t best = 0;
  int64_t best_cost = 0;
  for (int32_t sp = 1; sp <= max_span; ++sp) {
    n = pkv_decode_shared_plan(req_to_token, stride, seq_lens, batch, chunk, rows, sp, 1, priv ? 1 : 0, members,
                               skip, items, items_cap);
    if (n < 0) return n;
    const int64_t rounds = (n * hkv + resident_workgroups - 1) / resident_workgroups;
    const int64_t cost = rounds * (kItemFixed + (int64_t)sp * tiles_per_chunk);
    if (best == 0 || cost <= best_cost) {
      best = sp;
      best_cost = cost;
    }
  }
  if (best != max_span) {   // the outputs hold the last span's plan
    n = pkv_decode_shared_plan(req_to_token, stride, seq_lens, batch, chunk, rows, best, 1, priv ? 1 : 0, members,
                               skip, items, items_cap);
    if (n < 0) return n;
  }
  const int32_t fs = pkv_decode_first_split(skip, seq_lens, batch, chunk);
  if (fs < 0) return fs;
  *first_split = fs;
  return n;
}
