"""Throughput of the prefix-shared KV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload longctx_fp8|fewshot_bf16|decode_bf16|...]

A step is one pass of the whole hot path over one batch of synthetic input, with the
inputs (K/V/Q source rows) already resident in HBM:

  longctx_fp8 (default; the largest configuration on one GPU): 16 requests sharing a
  32,768-token prefix cached before the timed region, 1,024-token suffixes, GQA 64/8, d 128,
  fp8 e4m3 pool with per-head scales:
    rt_prepare_extend -> H2D tables -> kv_scatter (quantising) -> extend_attention
    -> 64 decode steps (rt_decode_step -> H2D -> kv_scatter -> decode_attention)
    -> rt_finish -> rt_evict of the batch's private tokens
  fewshot_bf16 (64 requests sharing a 1,800-token prefix that is cached before
  the timed region, suffixes U[150, 250], GQA 32/8, d 128, bf16, 200k-slot pool):
    rt_prepare_extend (match with split, lock, allocate, insert, relock for 64 requests)
    -> H2D tables -> kv_scatter of the suffix K/V -> extend_attention
    -> rt_decode_step (one slot per sequence) -> H2D -> kv_scatter -> decode_attention
    -> rt_finish (insert prompt + decoded token, unlock) -> rt_evict of the batch's private
       tokens (LRU leaves), so that every step meets the same cached state
  decode_bf16: one decode step of 512 sequences over 2,048-8,192-token contexts

Prints one JSON line.  `value` is query tokens (extend rows + decode rows) per second of
the whole step; `roofline` is the dominant kernel's achieved rate from HIP events on the
stream the library launches on, against MI355X's published peak; `cpu_baseline` is the
float64 CPU oracle on a bounded sample of the same workload.  Decode rates are reported on
three byte counts, never as one fraction above 1: the gathered bytes (each sequence's context
once; "effective" rate, which a shared prefix read once can push past the HBM peak), the
distinct K/V bytes of the step (a floor on what HBM must deliver) and, where the counters
were taken on the current kernels, the HBM bytes FETCH_SIZE/WRITE_SIZE measured.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "prefix_shared_kv_match_amd", "csrc")
# HBM bytes per launch of the extend kernel and per decode step (split phase, shared-prefix pass
# and reduce) of each workload, from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch; profiles/<workload>_kernels.md), scaled by what the same counters read for a
# plain 1 GiB device copy (FETCH x2.0, WRITE x1.0).  Each entry holds the hash of the kernel
# sources it was taken on; a changed kernel reports null.
TRAFFIC = {
    ("fewshot_bf16", "extend_attention"): dict(src_hash="fdaee6d5e67079b5", fetch_kib=205002.8, write_kib=102975.3),
    ("fewshot_bf16", "decode_attention"): dict(src_hash="78117e06109569ec", fetch_kib=30293.5 + 4291.0,
                                               write_kib=8494.2 + 512.0),
    ("decode_bf16", "decode_attention"): dict(src_hash="78117e06109569ec", fetch_kib=4215458.8 + 35224.7 + 23298.8,
                                              write_kib=39169.9 + 8704.0 + 4096.0),
    ("longctx_fp8", "extend_attention"): dict(src_hash="fdaee6d5e67079b5", fetch_kib=1471781.2, write_kib=319488.0),
    ("longctx_fp8", "decode_attention"): dict(src_hash="78117e06109569ec", fetch_kib=50994.1 + 9307.0,
                                              write_kib=18551.6 + 256.0),
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
# (warmup, timed) steps when not given: a few hundred ms of warmup for sub-millisecond steps,
# a handful of steps for the ones that run tens of milliseconds (one job, or a long-context
# extend with 64 decode steps)
DEFAULT_WARMUP_STEPS = {"fewshot_bf16": (200, 300), "decode_bf16": (40, 80), "longctx_fp8": (4, 10),
                        "multiturn_bf16": (5, 20), "tot_bf16": (5, 20)}
# the decode span is the split phase, the shared-prefix pass (in extend_attention.hip) and the
# reduce; its traffic entry is the sum over the three kernels per decode step
KERNEL_SOURCES = {"extend_attention": ["extend_attention.hip", "device.h"],
                  "decode_attention": ["decode_attention.hip", "extend_attention.hip", "device.h"]}


def kernel_src_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        h.update(n.encode())
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(workload: str, kernel: str):
    t = TRAFFIC.get((workload, kernel))
    if t is None or kernel_src_hash(kernel) != t["src_hash"]:
        return None
    return (t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default per workload: enough for a stable mean, a second or less)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default per workload: long enough for the GPU to leave its "
                         "idle clocks; a few milliseconds of warmup under-reports a sub-millisecond step)")
    ap.add_argument("--workload", default="longctx_fp8",
                    choices=["fewshot_bf16", "decode_bf16", "longctx_fp8", "multiturn_bf16", "tot_bf16"])
    ap.add_argument("--schedule", default="lpm", choices=["fcfs", "lpm"],
                    help="multiturn_bf16: batch order of the serve loop")
    ap.add_argument("--policy", default="lru", help="eviction policy of the radix tree (multiturn_bf16, tot_bf16)")
    ap.add_argument("--window", type=int, default=128, help="multiturn_bf16: waiting requests the scheduler sees")
    ap.add_argument("--batch", type=int, default=32, help="multiturn_bf16: requests per round")
    ap.add_argument("--chunk-budget", type=int, default=0,
                    help="fewshot_bf16: chunked prefill with at most this many new tokens per extend launch "
                         "(times the whole chunked job; 0 = the default one-batch step)")
    ap.add_argument("--plain-decode", action="store_true",
                    help="decode without the shared-prefix plan (every sequence gathers its whole context)")
    ap.add_argument("--decode-chunk", type=int, default=0,
                    help="tokens per decode split (a multiple of 64; 0 = the library's automatic choice)")
    ap.add_argument("--resident-workgroups", type=int, default=0,
                    help="shared-prefix decode: workgroups resident at once, by which the plan costs its item "
                         "span (0 = the engine's default)")
    ap.add_argument("--private-max-workgroups", type=int, default=-1,
                    help="shared-prefix decode: give the private tails to the shared-prefix kernel too when items "
                         "and tails need at most this many workgroups (-1 = the engine's default, 0 = never)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-batch", action="store_true",
                    help="long-context line: skip the extra key timing one step of the 512-sequence decode batch")
    ap.add_argument("--cpu-sample", type=int, default=64, help="requests in the oracle's timed sample")
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="extend rows per request in the oracle's timed sample (0 = all; -1 = 16 for the "
                         "long-context case, whose rows each cost ~2 GFLOP in float64, else all)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (reference for HBM byte counters)")
    return ap.parse_args()


class _NoSpan:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


class Timer:
    """HIP events on torch's current stream (the stream every library call is given).

    Events are created once, up front, and recycled: creating timing events inside the
    timed loop costs far more host time than the kernels it measures.  A timing event is
    not free on the GPU either (a few µs of queue time per record), so the timed loop records
    only the spans named in `live` (None: all)."""

    def __init__(self, torch, pool=4096):
        self.torch = torch
        self.free = [torch.cuda.Event(enable_timing=True) for _ in range(pool)]
        self.stream = torch.cuda.current_stream()
        self.acc = {}
        self.pending = []
        self.live = None

    def span(self, name):
        t = self
        if self.live is not None and name not in self.live:
            return _NoSpan()

        class _S:
            def __enter__(s):
                if len(t.free) < 2:
                    t.collect()
                s.a, s.b = t.free.pop(), t.free.pop()
                s.a.record(t.stream)

            def __exit__(s, *exc):
                s.b.record(t.stream)
                t.pending.append((name, s.a, s.b))
        return _S()

    def collect(self):
        self.torch.cuda.synchronize()
        for name, a, b in self.pending:
            ms, n = self.acc.get(name, (0.0, 0))
            self.acc[name] = (ms + a.elapsed_time(b), n + 1)
            self.free += [a, b]
        self.pending = []

    def reset(self):
        self.collect()
        self.acc = {}

    def avg_ms(self, name):
        ms, n = self.acc.get(name, (0.0, 0))
        return ms / n if n else float("nan")


def extend_flops(d, hq, prefix_lens, extend_lens):
    p = np.asarray(prefix_lens, dtype=np.float64)
    e = np.asarray(extend_lens, dtype=np.float64)
    pairs = float((e * p + e * (e + 1) / 2).sum())
    return 4.0 * d * hq * pairs, pairs


def kv_row_bytes(shape):
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}[shape.pool_dtype]
    return 2 * shape.hkv * shape.d * eb   # K and V of one token


class PathBench:
    """One workload's hot path; see the module docstring for what a step is."""

    CHUNK_ROWS = 65536   # setup scatter in chunks, so host memory stays bounded

    def __init__(self, torch, wl_name="fewshot_bf16", total_steps=64, shared_decode=True, decode_chunk=0):
        import workloads
        from prefix_shared_kv_match_amd.runtime import Engine
        self.torch = torch
        kw = {"steps": max(32, total_steps)} if wl_name == "decode_bf16" else {}
        self.wl = wl = workloads.make(wl_name, **kw)
        self.wl_kw = kw
        self.name = wl_name
        self.decode_only = not wl.extend_attention
        s = wl.shape
        self.eng = Engine(wl.pool_slots, s.hq, s.hkv, s.d, s.qo_dtype, s.pool_dtype, wl.free_order, "cuda",
                          wl.k_scale, wl.v_scale, wl.k_inv_scale, wl.v_inv_scale, s.sm_scale)
        eng = self.eng
        self.steps_dec = int(wl.decode_tokens.shape[0])
        self.stride = wl.max_len()
        batch = wl.batches[-1]
        B = len(batch)
        self.batch = batch
        self.timer = Timer(torch)
        # cache the shared prefixes (their K/V written to the pool) before anything is timed
        for r in wl.pre_insert:
            hb = eng.prepare([r.tokens], self.stride)
            self._scatter_rows(hb.new_slots, r.rows[hb.prefix_lens[0]:])
            eng.release(hb)
        from prefix_shared_kv_match_amd.runtime import flatten
        self.tokens = [r.tokens for r in batch]
        self.flat = flatten(self.tokens)            # the batch's token lists, concatenated once
        self.prompt_lens = [len(r.tokens) for r in batch]
        dev = torch.device("cuda")
        if self.decode_only:
            # the decode batch's contexts are prepared and written once; each step is one decode step
            hb = eng.prepare(self.tokens, self.stride)
            new_rows = np.concatenate([r.rows[p:] for r, p in zip(batch, hb.prefix_lens)])
            self._scatter_rows(hb.new_slots, new_rows)
            self.hb = hb
            self.r2t_dev = torch.from_numpy(hb.req_to_token.copy()).to(dev)
            self.max_len = self.stride
            self.step_i = 0
        else:
            pl = np.array([len(wl.pre_insert[0].tokens) if wl.pre_insert else 0] * B)
            self.new_rows = np.concatenate([r.rows[p:] for r, p in zip(batch, pl)])
            self.k_src, self.v_src = self._src(wl.values.k(self.new_rows)), self._src(wl.values.v(self.new_rows))
            self.q = self._src(wl.values.q(self.new_rows))
            self.o = torch.empty_like(self.q)
            self.full_tokens = flatten([np.concatenate([r.tokens, wl.decode_tokens[:, i]])
                                        for i, r in enumerate(batch)])
            self.max_len = max(self.prompt_lens) + self.steps_dec
        n_dec = self.steps_dec
        self.dk = [self._src(wl.values.k(wl.decode_rows[i])) for i in range(n_dec)]
        self.dv = [self._src(wl.values.v(wl.decode_rows[i])) for i in range(n_dec)]
        self.dq = [self._src(wl.values.q(wl.decode_rows[i])) for i in range(n_dec)]
        self.do = torch.empty_like(self.dq[0]) if n_dec else None
        if n_dec:
            self.ws, self.chunk = eng.decode_workspace(B, self.max_len, decode_chunk)
        # shared-prefix decode: which chunks the batch's sequences hold in common (made from the
        # host rows after the first decode slot is taken; valid while the sequences only grow)
        self.shared_decode = shared_decode
        self.plan = None
        if self.decode_only and shared_decode:
            self.plan = eng.decode_plan(self.hb.req_to_token, self.hb.seq_lens, self.chunk)
        self.last_tables = None
        self.host_prepare_s = 0.0

    def _src(self, a):
        t = self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        if self.wl.shape.qo_dtype == "bf16":
            t = t.to(self.torch.bfloat16)
        return t.to("cuda")

    def _scatter_rows(self, slots, rows):
        for lo in range(0, rows.size, self.CHUNK_ROWS):
            r = rows[lo:lo + self.CHUNK_ROWS]
            sl = self.torch.from_numpy(np.ascontiguousarray(slots[lo:lo + self.CHUNK_ROWS], dtype=np.int32)).to("cuda")
            self.eng.scatter(sl, self._src(self.wl.values.k(r)), self._src(self.wl.values.v(r)))
        self.torch.cuda.synchronize()

    def _decode_step(self, hb, r2t_dev, i):
        """rt_decode_step -> H2D (slots, lengths) -> append to the device table -> kv_scatter -> decode."""
        torch, eng, T = self.torch, self.eng, self.timer
        slots = eng.decode_alloc(hb)
        if self.decode_only or not self.shared_decode:
            slots_dev, seq_dev = eng.upload_decode(slots, hb.seq_lens)                # async copy
        else:
            if i == 0:      # the batch's shared chunks (host); sent with every step's slots
                self.plan_host = eng.decode_plan(hb.req_to_token, hb.seq_lens, self.chunk, upload=False)
            if self.plan_host is None:
                slots_dev, seq_dev = eng.upload_decode(slots, hb.seq_lens)
                self.plan = None
            else:
                slots_dev, seq_dev, self.plan = eng.upload_decode(slots, hb.seq_lens, self.plan_host)
        eng.append_slots(r2t_dev, seq_dev, slots_dev)
        with T.span("kv_scatter_decode"):
            eng.scatter(slots_dev, self.dk[i], self.dv[i])
        with T.span("decode_attention"):
            eng.decode(self.dq[i], r2t_dev, seq_dev, self.max_len, self.ws, self.chunk, self.do, plan=self.plan,
                       seq_lens_host=hb.seq_lens)

    def step(self):
        import prefix_shared_kv_match_amd as pkv
        eng, T = self.eng, self.timer
        if self.decode_only:
            i = self.step_i % self.steps_dec
            self.step_i += 1
            if int(self.hb.seq_lens.max()) >= self.stride:
                raise RuntimeError("decode bench ran past the table stride; use fewer steps")
            self._decode_step(self.hb, self.r2t_dev, i)
            self.last_tables = self.hb
            return self.hb.n
        th = time.perf_counter()
        hb = eng.prepare_staged(self.flat, self.stride)                  # host: match/lock/alloc/insert
        self.host_prepare_s += time.perf_counter() - th
        dt = eng.device_tables(hb, staged=True)                          # H2D tables + plan (async)
        with T.span("kv_scatter"):
            eng.scatter(dt["new_slots"], self.k_src, self.v_src)
        with T.span("extend_attention"):
            eng.extend(dt, self.q, self.o)
        for i in range(self.steps_dec):
            self._decode_step(hb, dt["req_to_token"], i)
        if self.steps_dec:
            eng.finish(hb, self.full_tokens, self.prompt_lens)
        else:
            eng.release(hb)
        n_private = int(hb.extend_lens.sum()) + self.steps_dec * hb.n
        pkv.rt_evict(eng.tree, n_private)                                # keep only the shared prefix cached
        self.last_tables = hb
        return int(hb.extend_lens.sum()) + self.steps_dec * hb.n


class JobBench:
    """A whole multi-round job per step, with every round's inputs resident in HBM.

    multiturn_bf16: the serve loop over all 1,024 arrivals (rt_schedule_longest_prefix or
    arrival order, rt_prepare_extend_prio, staged tables, kv_scatter, extend_attention,
    rt_release per round).  tot_bf16: the four tree levels in order, then 16 decode steps
    of the 256 leaves and rt_finish.  A step ends by evicting what it inserted (the ToT
    root stays cached), so every step meets the same tree."""

    def __init__(self, torch, a):
        import workloads
        from prefix_shared_kv_match_amd import runtime
        from prefix_shared_kv_match_amd.runtime import Engine
        self.torch, self.rt = torch, runtime
        kw = {"decode_steps": 0} if a.workload == "fewshot_bf16" else {}
        self.wl = wl = workloads.make(a.workload, **kw)
        self.name, self.a = a.workload, a
        s = wl.shape
        self.eng = eng = Engine(wl.pool_slots, s.hq, s.hkv, s.d, s.qo_dtype, s.pool_dtype, wl.free_order, "cuda",
                                sm_scale=s.sm_scale, policy=a.policy)
        if a.resident_workgroups:
            eng.RESIDENT_WORKGROUPS = a.resident_workgroups
        if a.private_max_workgroups >= 0:
            eng.PRIVATE_MAX_WORKGROUPS = a.private_max_workgroups
        self.stride = wl.max_len()
        self.timer = Timer(torch)
        self.decode_only = False
        # every canonical K/V/Q row on the device (bf16), so a round's inputs are one gather away
        self.K = self._table(workloads.TAG_K)
        self.V = self._table(workloads.TAG_V)
        self.Q = self._table(workloads.TAG_Q)
        self.root_len = 0
        for r in wl.pre_insert:
            hb = eng.prepare([r.tokens], self.stride)
            self._scatter_rows(hb.new_slots, r.rows[hb.prefix_lens[0]:])
            eng.release(hb)
            self.root_len += len(r.tokens)
        self.arr = [x for b in wl.batches for x in b]
        # dry run of the host steps on a twin tree: which rows each round extends
        twin = runtime.rt_create_policy(wl.pool_slots, wl.free_order, a.policy)
        try:
            for r in wl.pre_insert:
                runtime.rt_release(twin, runtime.prepare(twin, [r.tokens], self.stride).last_nodes)
            self.plan = self._host_rounds(twin, None)
        finally:
            runtime.rt_destroy(twin)
        self.inputs = []
        for pick, pl, ends in self.plan:
            rows = np.concatenate([self.arr[i].rows[p:e] for i, p, e in zip(pick, pl, ends)]) if pick else np.zeros(0)
            idx = torch.from_numpy(rows.astype(np.int64)).cuda()
            self.inputs.append((self.K.index_select(0, idx), self.V.index_select(0, idx), self.Q.index_select(0, idx)))
        self.o = torch.empty((max(x[2].shape[0] for x in self.inputs), s.hq, s.d), dtype=torch.bfloat16, device="cuda")
        self.steps_dec = int(wl.decode_tokens.shape[0])
        if self.steps_dec:
            last = wl.batches[-1]
            B = len(last)
            dr = torch.from_numpy(wl.decode_rows.astype(np.int64)).cuda()
            self.dk = [self.K.index_select(0, dr[i]) for i in range(self.steps_dec)]
            self.dv = [self.V.index_select(0, dr[i]) for i in range(self.steps_dec)]
            self.dq = [self.Q.index_select(0, dr[i]) for i in range(self.steps_dec)]
            self.do = torch.empty_like(self.dq[0])
            self.max_len = max(len(r.tokens) for r in last) + self.steps_dec
            self.ws, self.chunk = eng.decode_workspace(B, self.max_len, a.decode_chunk)
            self.full_tokens = [np.concatenate([r.tokens, wl.decode_tokens[:, i]]) for i, r in enumerate(last)]
            self.prompt_lens = [len(r.tokens) for r in last]
        torch.cuda.synchronize()
        self.flops = 0.0
        self.ext_tokens = 0
        for pick, pl, ends in self.plan:
            el = [e - p for p, e in zip(pl, ends)]
            self.flops += extend_flops(s.d, s.hq, pl, el)[0]
            self.ext_tokens += int(sum(el))
        self.prompt_tokens = sum(len(r.tokens) for r in self.arr)
        # tokens served from the cache: each request's first prefix length (later chunks of a
        # request reuse its own earlier chunks, which were computed in this job)
        first = {}
        for pick, pl, _ in self.plan:
            for i, p in zip(pick, pl):
                first.setdefault(i, p)
        self.cached_tokens = sum(first.values())

    def _table(self, tag):
        full = self.wl.values.full(tag)
        t = self.torch.from_numpy(full).to("cuda").to(self.torch.bfloat16)
        del full
        return t

    def _scatter_rows(self, slots, rows):
        torch = self.torch
        idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()
        sl = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).cuda()
        self.eng.scatter(sl, self.K.index_select(0, idx), self.V.index_select(0, idx))
        torch.cuda.synchronize()

    def _host_rounds(self, tree, on_round):
        """Runs the job's host steps on `tree`; on_round(k, host_batch) does round k's device work.
        Returns [(request indices, prefix lengths, end positions)] per round."""
        rt, wl, a = self.rt, self.wl, self.a
        out = []
        if self.name == "fewshot_bf16":   # chunked prefill of the 64-request batch
            def cb(reqs, ends, hb):
                if on_round is not None:
                    on_round(len(out), hb)
                out.append((list(reqs), hb.prefix_lens.tolist(), list(ends)))
            rt.chunked_prefill(tree, [r.tokens for r in self.arr], a.chunk_budget, self.stride, on_launch=cb)
            return out
        if self.name == "multiturn_bf16":
            def cb(pick, hb):
                if on_round is not None:
                    on_round(len(out), hb)
                out.append((list(pick), hb.prefix_lens.tolist(), [len(self.arr[i].tokens) for i in pick]))
            rt.serve(tree, [r.tokens for r in self.arr], [r.after for r in self.arr], a.schedule, a.batch, a.window,
                     self.stride, priorities=[r.priority for r in self.arr], on_batch=cb)
            return out
        base = 0
        for bi, batch in enumerate(wl.batches):
            hb = rt.prepare(tree, [r.tokens for r in batch], self.stride)
            if on_round is not None:
                on_round(len(out), hb)
            out.append((list(range(base, base + len(batch))), hb.prefix_lens.tolist(), [len(r.tokens) for r in batch]))
            base += len(batch)
            if bi < len(wl.batches) - 1 or not wl.decode_tokens.shape[0]:
                rt.rt_release(tree, hb.last_nodes)
            else:
                self._last_hb = hb
        return out

    def _round(self, k, hb):
        eng, T = self.eng, self.timer
        pick, pl, _ = self.plan[k]
        if hb.prefix_lens.tolist() != pl:
            raise RuntimeError(f"round {k} matched differently from the planning run")
        dt = eng.device_tables(hb, staged=True)
        ks, vs, qs = self.inputs[k]
        if hb.n_new:
            with T.span("kv_scatter"):
                eng.scatter(dt["new_slots"], ks, vs)
            with T.span("extend_attention"):
                eng.extend(dt, qs, self.o[:hb.n_new])
        self._last_dt = dt

    def step(self):
        import prefix_shared_kv_match_amd as pkv
        eng, T = self.eng, self.timer
        self._host_rounds(eng.tree, self._round)
        n = self.ext_tokens
        if self.steps_dec:
            hb = self._last_hb
            r2t = self._last_dt["req_to_token"]
            plan_host = plan = None
            for i in range(self.steps_dec):
                slots = eng.decode_alloc(hb)
                if i == 0 and not self.a.plain_decode:     # the batch's shared chunks, on the host
                    plan_host = eng.decode_plan(hb.req_to_token, hb.seq_lens, self.chunk, upload=False)
                if plan_host is None:
                    slots_dev, seq_dev = eng.upload_decode(slots, hb.seq_lens)
                else:                                       # sent with every step's slots
                    slots_dev, seq_dev, plan = eng.upload_decode(slots, hb.seq_lens, plan_host)
                eng.append_slots(r2t, seq_dev, slots_dev)
                with T.span("kv_scatter_decode"):
                    eng.scatter(slots_dev, self.dk[i], self.dv[i])
                with T.span("decode_attention"):
                    eng.decode(self.dq[i], r2t, seq_dev, self.max_len, self.ws, self.chunk, self.do, plan=plan)
            eng.finish(hb, self.full_tokens, self.prompt_lens)
            n += self.steps_dec * hb.n
        pkv.rt_evict(eng.tree, pkv.rt_evictable_size(eng.tree) - self.root_len)
        return n

    def host_hit_rates(self):
        """Cached-prefix share of the prompt tokens for every eviction policy x batch order (host only)."""
        rt = self.rt
        out = {}
        for order in ("fcfs", "lpm"):
            for pol in ("lru", "lfu", "slru", "fifo", "mru", "filo", "priority"):
                t = rt.rt_create_policy(self.wl.pool_slots, self.wl.free_order, pol)
                try:
                    res = rt.serve(t, [r.tokens for r in self.arr], [r.after for r in self.arr], order, self.a.batch,
                                   self.a.window, self.stride, priorities=[r.priority for r in self.arr])
                finally:
                    rt.rt_destroy(t)
                cached = sum(int(hb.prefix_lens.sum()) for _, hb in res)
                prio_c = sum(int(hb.prefix_lens[j]) for p, hb in res for j, i in enumerate(p) if self.arr[i].priority)
                prio_t = sum(len(r.tokens) for r in self.arr if r.priority)
                out[f"{order}/{pol}"] = {"all": round(cached / self.prompt_tokens, 4),
                                         "priority_class": round(prio_c / max(prio_t, 1), 4)}
        return out


def practical_hbm_gbps(torch, mib=4096, reps=5):
    """The library's streaming-read kernel (pkv_stream_read) over `mib` MiB, far beyond the
    256 MB last-level cache, best of `reps`: the read rate HBM delivers to a plain kernel on
    this GPU, next to the published 8 TB/s."""
    import prefix_shared_kv_match_amd as pkv
    lib = pkv.lib()
    buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(int(lib.pkv_stream_read_words()), dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    best = float("inf")
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pkv.check(lib.pkv_stream_read(buf.data_ptr(), buf.numel() * 4, out.data_ptr(), st))
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf, out
    torch.cuda.empty_cache()
    return mib * (1 << 20) / best / 1e6


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main_job(a, torch):
    import prefix_shared_kv_match_amd as pkv
    b = JobBench(torch, a)
    wl, s = b.wl, b.wl.shape
    b.timer.live = {"extend_attention"}      # the only span recorded in the timed loop
    for _ in range(a.warmup):
        b.step()
    b.timer.reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tokens = 0
    for _ in range(a.steps):
        tokens += b.step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    b.timer.collect()
    live_acc = dict(b.timer.acc)
    extra = min(3, a.steps) if b.steps_dec else 0     # untimed jobs for the decode spans
    b.timer.live = None
    b.timer.reset()
    for _ in range(extra):
        b.step()
    b.timer.collect()
    b.timer.acc.update(live_acc)
    ext_ms, n_ext = b.timer.acc.get("extend_attention", (0.0, 0))
    ext_ms_job = ext_ms / a.steps
    kernels = {"extend_attention": {"ms_per_job": ext_ms_job, "launches_per_job": n_ext // a.steps,
                                    "tflops": b.flops / ext_ms_job / 1e9,
                                    "frac_mfma": b.flops / ext_ms_job / 1e9 / PEAK_BF16_TFLOPS}}
    if b.steps_dec:
        dm, dn = b.timer.acc.get("decode_attention", (0.0, 0))
        kernels["decode_attention"] = {"ms": dm / max(dn, 1)}
    out = {
        "metric": "served prompt tokens/s over a whole multi-round job (radix reuse + extend + decode)",
        "value": b.prompt_tokens * a.steps / el, "unit": "prompt tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": el / a.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "requests": len(b.arr), "rounds": len(b.plan), "policy": a.policy,
                   "schedule": a.schedule if wl.name == "multiturn_bf16" else (
                       f"chunked prefill, {a.chunk_budget} new tokens per launch" if wl.name == "fewshot_bf16"
                       else "levels in order"),
                   "window": a.window if wl.name == "multiturn_bf16" else None,
                   "hq": s.hq, "hkv": s.hkv, "head_dim": s.d, "pool_slots": wl.pool_slots,
                   "capacity": int(len(wl.free_order))},
        "prompt_tokens_per_job": b.prompt_tokens, "cached_tokens_per_job": b.cached_tokens,
        "hit_rate": b.cached_tokens / b.prompt_tokens, "query_tokens_per_s": tokens / el,
        "roofline": {"bound": "mfma", "kernel": "extend_attention", "achieved": b.flops / ext_ms_job / 1e9,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": b.flops / ext_ms_job / 1e9 / PEAK_BF16_TFLOPS, "traffic": None},
        "kernels": kernels,
        "library": os.path.relpath(pkv._capi.LIB_PATH, ROOT),
    }
    if wl.name == "multiturn_bf16":
        out["host_hit_rates"] = b.host_hit_rates()
    print(json.dumps(out), flush=True)
    return 0


def decode_batch_key(torch, warmup=20, steps=40):
    """One decode step of the 512-sequence decode batch (contexts U[2048, 8192], 16 shared
    1,024-token prefixes, bf16): the HBM-bound decode case, timed like the decode workload's
    own line (HIP events around the decode span on the launch stream, after warmup steps).
    Bytes are those of the last timed step's contexts."""
    b = PathBench(torch, "decode_bf16", warmup + steps)
    b.timer.live = {"decode_attention"}
    for _ in range(warmup):
        b.step()
    b.timer.reset()
    torch.cuda.synchronize()
    for _ in range(steps):
        b.step()
    torch.cuda.synchronize()
    b.timer.collect()
    hb, s = b.last_tables, b.wl.shape
    ms = b.timer.avg_ms("decode_attention")
    kv_tok = kv_row_bytes(s)
    uniq = float(np.unique(np.concatenate([hb.req_to_token[i, :hb.seq_lens[i]] for i in range(hb.n)])).size) * kv_tok
    hbm = traffic_bytes("decode_bf16", "decode_attention")
    return {"workload": "decode_bf16", "sequences": int(hb.n), "steps": steps, "ms": ms,
            "unique_kv_bytes": uniq, "unique_gbps": uniq / ms / 1e6, "frac_hbm_unique": uniq / ms / 1e6 / PEAK_HBM_GBPS,
            "hbm_bytes": hbm, "hbm_gbps": None if hbm is None else hbm / ms / 1e6,
            "frac_hbm": None if hbm is None else hbm / ms / 1e6 / PEAK_HBM_GBPS}


def _cpu_worker(job):
    """One process of the CPU baseline: the oracle over its share of the sample (one BLAS
    thread), repeated until at least min_seconds of work; returns (query tokens, seconds)."""
    name, kw, decode_only, items, min_seconds = job
    import workloads
    from oracle import attention as oa
    wl = workloads.make(name, **kw)
    reqs = wl.batches[-1]
    n, t0 = 0, time.perf_counter()
    while True:
        for it in items:
            if decode_only:
                i, steps = it
                oa.decode_row(wl, np.concatenate([reqs[i].rows, wl.decode_rows[:steps, i]]))
                n += 1
            else:
                i, p, pos = it
                oa.extend_rows(wl, reqs[i], p, sample=pos)
                n += len(pos)
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return n, dt


def cpu_baseline(wl, wl_kw, hb, n_req, decode_only=False, steps_done=0, min_seconds=10.0, rows_per_req=0,
                 max_workers=16):
    """The float64 oracle on a bounded sample in a pool of processes with one BLAS thread each
    (at most max_workers, the host cores a one-GPU job gets): the extend rows of the first n_req
    requests (with rows_per_req > 0, that many rows of each, a seeded sample that holds the
    first and last), or (decode workload) the newest decode row of the first n_req sequences
    over their whole current context.  Work is cut into (request, rows) units dealt round-robin
    to the processes; each repeats its share until min_seconds have passed, and the rate is the
    tokens done over the longest process's time."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    reqs = wl.batches[-1][:n_req]
    workers = max(1, min(max_workers, os.cpu_count() or 1))
    rng = np.random.default_rng(0)
    units = []
    for i, r in enumerate(reqs):
        if decode_only:
            units.append((i, int(steps_done)))
            continue
        p = int(hb.prefix_lens[i])
        pos = np.arange(p, len(r.tokens))
        if rows_per_req and pos.size > rows_per_req:
            mid = rng.choice(pos[1:-1], size=rows_per_req - 2, replace=False)
            pos = np.sort(np.concatenate([[pos[0], pos[-1]], mid]))
        parts = max(1, min(pos.size, -(-workers // max(len(reqs), 1))))
        units += [(i, p, c) for c in np.array_split(pos, parts) if c.size]
    workers = min(workers, len(units))
    shares = [units[w::workers] for w in range(workers)]
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    os.environ.update({k: "1" for k in saved})
    try:
        with ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("spawn")) as ex:
            res = list(ex.map(_cpu_worker, [(wl.name, wl_kw, decode_only, sh, min_seconds) for sh in shares]))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    rows = sum(n for n, _ in res)
    dt = max(t for _, t in res)
    what = "newest decode row" if decode_only else (
        f"{rows_per_req} sampled extend rows" if rows_per_req else "extend rows")
    return {"value": rows / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"float64 numpy oracle in {workers} processes of one BLAS thread each ({cpu_model()}): {what} "
                      f"of the first {len(reqs)} of {len(wl.batches[-1])} "
                      f"{'sequences' if decode_only else 'requests'} over their full contexts, cut into "
                      f"{len(units)} (request, rows) units; {rows} query tokens, the longest process "
                      f"{dt:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported (the library runs one GPU per "
              f"process and has no multi-GPU path)", file=sys.stderr)
        return 2
    dw, ds = DEFAULT_WARMUP_STEPS[a.workload]
    a.warmup = dw if a.warmup is None else a.warmup
    a.steps = ds if a.steps is None else a.steps
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    import prefix_shared_kv_match_amd as pkv
    pkv.lib()
    if a.workload in ("multiturn_bf16", "tot_bf16") or (a.workload == "fewshot_bf16" and a.chunk_budget > 0):
        return main_job(a, torch)
    extra = min(30, a.steps)      # untimed steps after the timed ones, for the other kernels' spans
    b = PathBench(torch, a.workload, a.warmup + a.steps + extra, shared_decode=not a.plain_decode,
                  decode_chunk=a.decode_chunk)
    if a.resident_workgroups or a.private_max_workgroups >= 0:
        if a.resident_workgroups:
            b.eng.RESIDENT_WORKGROUPS = a.resident_workgroups
        if a.private_max_workgroups >= 0:
            b.eng.PRIVATE_MAX_WORKGROUPS = a.private_max_workgroups
        if b.plan is not None:      # a decode-only batch planned at construction: plan again
            b.plan = b.eng.decode_plan(b.hb.req_to_token, b.hb.seq_lens, b.chunk)
    wl = b.wl
    if a.copy_calib_mib:
        n = a.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the timed loop records events around the dominant kernel only
    dominant = "extend_attention" if wl.extend_attention else "decode_attention"
    b.timer.live = {dominant}
    for _ in range(a.warmup):
        b.step()
    b.timer.reset()
    b.host_prepare_s = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tokens = 0
    for _ in range(a.steps):
        tokens += b.step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    b.timer.collect()
    live_acc = dict(b.timer.acc)
    # the tables the timed steps ran on (the extra steps below overwrite the staging buffers
    # and, for the decode workload, grow the contexts)
    import dataclasses
    lt = b.last_tables
    timed_tables = dataclasses.replace(lt, req_to_token=lt.req_to_token.copy(), seq_lens=lt.seq_lens.copy(),
                                       prefix_lens=lt.prefix_lens.copy(), extend_lens=lt.extend_lens.copy())
    timed_step_i = b.step_i if b.decode_only else 0
    # then a few untimed steps with every span, for the other kernels' durations
    b.timer.live = None
    b.timer.reset()
    host_prepare_s = b.host_prepare_s
    for _ in range(extra):
        b.step()
    b.timer.collect()
    b.timer.acc.update(live_acc)
    b.host_prepare_s = host_prepare_s
    hbm_practical = practical_hbm_gbps(torch)
    hb = timed_tables
    s = wl.shape
    flops, pairs = extend_flops(s.d, s.hq, hb.prefix_lens, hb.extend_lens)
    kv_tok = kv_row_bytes(s)
    ext_ms = b.timer.avg_ms("extend_attention")
    dec_ms = b.timer.avg_ms("decode_attention")
    gathered_ext = float((hb.prefix_lens.astype(np.float64) + hb.extend_lens).sum()) * kv_tok
    kernels = {}
    if wl.extend_attention:
        kernels["extend_attention"] = {
            "ms": ext_ms, "tflops": flops / ext_ms / 1e9, "frac_mfma": flops / ext_ms / 1e9 / PEAK_BF16_TFLOPS,
            "kv_gathered_gbps": gathered_ext / ext_ms / 1e6, "flops": flops, "pairs": pairs,
            "query_tokens": int(hb.extend_lens.sum()),
            "q_o_bytes": 2.0 * float(hb.extend_lens.sum()) * s.hq * s.d * (4 if s.qo_dtype == "f32" else 2),
            "unique_kv_bytes": float(np.unique(np.concatenate(
                [hb.req_to_token[i, :hb.seq_lens[i]] for i in range(hb.n)])).size) * kv_tok,
            "host_prepare_ms": b.host_prepare_s / a.steps * 1e3}
    if b.steps_dec:
        ctx = hb.seq_lens.astype(np.float64)
        dec_bytes = float(ctx.sum()) * kv_tok
        # the distinct K/V rows of the step: the bytes HBM must deliver at least once (the
        # gathered bytes count a shared prefix once per sequence)
        uniq = float(np.unique(np.concatenate([hb.req_to_token[i, :hb.seq_lens[i]] for i in range(hb.n)])).size)
        hbm = traffic_bytes(wl.name, "decode_attention")
        kernels["decode_attention"] = {
            "ms": dec_ms, "chunk": int(getattr(b, "chunk", 0)),
            "gathered_bytes": dec_bytes, "effective_gbps": dec_bytes / dec_ms / 1e6,
            "unique_kv_bytes": uniq * kv_tok, "unique_gbps": uniq * kv_tok / dec_ms / 1e6,
            "frac_hbm_unique": uniq * kv_tok / dec_ms / 1e6 / PEAK_HBM_GBPS,
            "hbm_bytes": hbm, "hbm_gbps": None if hbm is None else hbm / dec_ms / 1e6,
            "frac_hbm": None if hbm is None else hbm / dec_ms / 1e6 / PEAK_HBM_GBPS,
            "frac_hbm_practical": None if hbm is None else hbm / dec_ms / 1e6 / hbm_practical,
            "tflops": 4.0 * s.d * s.hq * float(ctx.sum()) / dec_ms / 1e9,
            "note": "effective_gbps counts each sequence's whole context (a shared prefix once per sequence) and "
                    "can exceed the HBM peak when shared chunks are read once; frac_hbm is on the HBM bytes the "
                    "counters measured (null until taken on the current kernels); frac_hbm_unique on the "
                    "distinct K/V bytes, a floor on HBM traffic"}
    sc_name = "kv_scatter_decode" if b.decode_only else "kv_scatter"
    sc_ms = b.timer.avg_ms(sc_name)
    n_new = hb.n if b.decode_only else int(hb.extend_lens.sum())
    src_b = 2 * s.hkv * s.d * (4 if s.qo_dtype == "f32" else 2)
    kernels["kv_scatter"] = {"ms": sc_ms, "gbps": n_new * (src_b + kv_tok) / sc_ms / 1e6}
    basis = None
    if wl.extend_attention:
        dom, bound = "extend_attention", "mfma"
        achieved, peak, unit = kernels[dom]["tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"
        basis = "algorithmic FLOPs 4*d*hq*sum(e*p + e(e+1)/2) from the tree's (p, e) / extend time"
    else:
        dom, bound = "decode_attention", "hbm"
        k = kernels[dom]
        peak, unit = PEAK_HBM_GBPS, "GB/s"
        if k["hbm_gbps"] is not None:
            achieved, basis = k["hbm_gbps"], "HBM bytes measured by FETCH_SIZE/WRITE_SIZE / decode time"
        else:
            achieved, basis = k["unique_gbps"], "distinct K/V bytes of the step / decode time (counters not taken)"
    out = {
        "metric": "extend+decode attention tokens/s, TFLOP/s & KV GB/s vs MI355X roofline",
        "value": tokens / el, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": el / a.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if s.qo_dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "requests": hb.n, "query_tokens_per_step": tokens // a.steps,
                   "hq": s.hq, "hkv": s.hkv, "head_dim": s.d, "pool_dtype": s.pool_dtype,
                   "pool_slots": wl.pool_slots, "decode_steps_per_step": 1 if b.decode_only else b.steps_dec},
        "roofline": {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic_bytes(wl.name, dom), "basis": basis},
        "kernels": kernels,
        "kernel_timing": f"{dom}: HIP events in every timed step (the only span recorded there); the other "
                         f"kernels: HIP events over {extra} untimed steps after the timed ones",
        "hbm_practical_read_gbps": hbm_practical,
        "library": os.path.relpath(pkv._capi.LIB_PATH, ROOT),
    }
    wl_kw, decode_only = b.wl_kw, b.decode_only
    if wl.name == "longctx_fp8" and not a.no_decode_batch:
        del b
        torch.cuda.empty_cache()
        out["decode_batch"] = decode_batch_key(torch)
    if not a.no_cpu_baseline:
        rows = a.cpu_rows if a.cpu_rows >= 0 else (16 if wl.name == "longctx_fp8" else 0)
        out["cpu_baseline"] = cpu_baseline(wl, wl_kw, hb, a.cpu_sample, decode_only, timed_step_i,
                                           rows_per_req=rows)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
