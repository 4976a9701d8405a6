"""Seeded synthetic inputs shared by the HIP path, its tests, the bench and the oracle.

This module draws token sequences, arrival orders and the K/V/Q value tables.
It computes none of the method: no prefix matching, no slot allocation, no
attention and no quantisation (the fp8 scales below are calibration inputs,
i.e. per-head maxima of the drawn values, not the quantiser itself).

Value model.  In a real model the K/V of a token depends on the whole token
path before it, so a prefix cache may only reuse a row when the full token
path matches.  Here every token position of every request maps to a row of a
canonical table; the rows are laid out per *segment* (a run of tokens that is
always seen together: a shared prefix, one suffix, one chat turn), and the
segments form a tree.  Siblings in that tree are drawn with distinct first
tokens, so two token sequences share a prefix exactly as long as their
segment paths do, and equal token paths always carry equal rows.

Values are N(0,1) float32 from numpy PCG64 streams seeded per (config seed,
table, block of 512 rows), so any row can be produced on its own and the full
tables can be drawn in parallel.  They are then rounded (round to nearest
even) to the precision they are stored in: float32 for the fp32 case, bf16
for every other case (including the fp8-pool case, whose kv_scatter source is
bf16).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Tuple

import numpy as np

BLOCK_ROWS = 512
TAG_K, TAG_V, TAG_Q = 11, 12, 13
LLAMA3_VOCAB = 128256


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Inputs here are finite normals, so no NaN/Inf handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Shape:
    hq: int
    hkv: int
    d: int
    qo_dtype: str      # "f32" or "bf16": dtype of q, o and of the kv_scatter source
    pool_dtype: str    # "f32", "bf16" or "fp8_e4m3"
    sm_scale: float

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclasses.dataclass
class Request:
    tokens: np.ndarray   # int32 [L]
    rows: np.ndarray     # int64 [L]: canonical value row of each position
    tag: str = ""        # human readable origin, e.g. "conv17/turn3"
    after: int = -1      # arrival index of a request that must be served first (previous turn), -1 none
    priority: int = 0    # importance class a caller assigns (read only by the priority eviction policy)


class ValueTable:
    """Canonical K, V and Q rows.  K/V rows are [hkv, d]; Q rows are [hq, d]."""

    def __init__(self, seed: int, n_rows: int, shape: Shape):
        self.seed = int(seed)
        self.n_rows = int(n_rows)
        self.shape = shape
        self._cache: Dict[Tuple[int, int], np.ndarray] = {}

    def _width(self, tag: int) -> int:
        s = self.shape
        return (s.hq if tag == TAG_Q else s.hkv) * s.d

    def _round(self, a: np.ndarray) -> np.ndarray:
        return a if self.shape.qo_dtype == "f32" else round_to_bf16(a)

    def _gen_block(self, tag: int, b: int) -> np.ndarray:
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, tag, b]))
        a = rng.standard_normal((BLOCK_ROWS, self._width(tag)), dtype=np.float32)
        return self._round(a)

    def _block(self, tag: int, b: int) -> np.ndarray:
        key = (tag, b)
        blk = self._cache.get(key)
        if blk is None:
            if len(self._cache) > 256:
                self._cache.clear()
            blk = self._gen_block(tag, b)
            self._cache[key] = blk
        return blk

    def _rows(self, tag: int, rows: np.ndarray) -> np.ndarray:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        if rows.size and (rows.min() < 0 or rows.max() >= self.n_rows):
            raise IndexError("value row out of range")
        out = np.empty((rows.size, self._width(tag)), dtype=np.float32)
        blocks = rows // BLOCK_ROWS
        ub = np.unique(blocks)
        if ub.size > 32:
            # many blocks: draw them in parallel without caching
            order = np.argsort(blocks, kind="stable")
            bounds = np.searchsorted(blocks[order], ub, side="left").tolist() + [rows.size]

            def fill(i: int) -> None:
                sel = order[bounds[i]:bounds[i + 1]]
                b = int(ub[i])
                out[sel] = self._gen_block(tag, b)[rows[sel] - b * BLOCK_ROWS]

            with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
                list(ex.map(fill, range(ub.size)))
        else:
            for b in ub:
                sel = np.nonzero(blocks == b)[0]
                out[sel] = self._block(tag, int(b))[rows[sel] - b * BLOCK_ROWS]
        h = self.shape.hq if tag == TAG_Q else self.shape.hkv
        return out.reshape(rows.size, h, self.shape.d)

    def k(self, rows) -> np.ndarray:
        return self._rows(TAG_K, rows)

    def v(self, rows) -> np.ndarray:
        return self._rows(TAG_V, rows)

    def q(self, rows) -> np.ndarray:
        return self._rows(TAG_Q, rows)

    def full(self, tag: int, threads: Optional[int] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
        """Every row of one table, drawn block-parallel; float32 [n_rows, h, d]."""
        n_blocks = (self.n_rows + BLOCK_ROWS - 1) // BLOCK_ROWS
        w = self._width(tag)
        if out is None:
            out = np.empty((self.n_rows, w), dtype=np.float32)
        else:
            out = out.reshape(self.n_rows, w)

        def fill(b: int) -> None:
            lo = b * BLOCK_ROWS
            hi = min(self.n_rows, lo + BLOCK_ROWS)
            out[lo:hi] = self._gen_block(tag, b)[: hi - lo]

        threads = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_blocks)))
        h = self.shape.hq if tag == TAG_Q else self.shape.hkv
        return out.reshape(self.n_rows, h, self.shape.d)


class StressValues(ValueTable):
    """A value table with a sharpened softmax and planted keys, for stress cases.

    Every Q row is replaced by q_mul * q + beta * u_g (per query head, u_g a fixed unit vector of
    its kv head drawn from the seed), and the K rows listed in ``plant_rows`` by gamma * u_g, all
    rounded to the stored precision again.  A planted key then meets every query with a logit
    of about gamma * (q_mul * <q, u> + beta) * scale, far above the others when gamma and beta are
    large: a query that sees one after other keys must move its running maximum.  Input
    construction only (scaling and replacing rows of the drawn tables)."""

    def __init__(self, base: ValueTable, q_mul: float = 1.0, beta: float = 0.0, gamma: float = 0.0,
                 plant_rows=()):
        super().__init__(base.seed, base.n_rows, base.shape)
        self.q_mul, self.beta, self.gamma = float(q_mul), float(beta), float(gamma)
        self.plant = np.unique(np.asarray(plant_rows, dtype=np.int64))
        rng = np.random.default_rng(np.random.SeedSequence([base.seed, 97]))
        u = rng.standard_normal((base.shape.hkv, base.shape.d))
        self.u = (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)

    def _gen_block(self, tag: int, b: int) -> np.ndarray:
        a = super()._gen_block(tag, b)
        s = self.shape
        if tag == TAG_Q and (self.q_mul != 1.0 or self.beta != 0.0):
            g = np.arange(s.hq) // s.group
            a = (a.reshape(BLOCK_ROWS, s.hq, s.d) * np.float32(self.q_mul)
                 + np.float32(self.beta) * self.u[g][None]).reshape(BLOCK_ROWS, -1)
            a = self._round(a.astype(np.float32))
        elif tag == TAG_K and self.plant.size:
            rows = b * BLOCK_ROWS + np.arange(BLOCK_ROWS)
            hit = np.isin(rows, self.plant)
            if hit.any():
                a = a.copy()
                a[hit] = self._round((np.float32(self.gamma) * self.u).reshape(1, -1))
        return a


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    shape: Shape
    pool_slots: int
    free_order: np.ndarray            # int32 [capacity]: the allocator's initial free list, head first
    pre_insert: List[Request]         # inserted one by one (match, alloc, insert, scatter, unlock) before the batches
    batches: List[List[Request]]      # extend batches, in arrival order
    extend_attention: bool            # False: batches are only prepared and scattered (decode setup)
    decode_tokens: np.ndarray         # int32 [steps, B] for the sequences of the last batch (steps may be 0)
    decode_rows: np.ndarray           # int64 [steps, B]
    values: ValueTable
    k_scale: Optional[np.ndarray] = None   # float32 [hkv], fp8 pool only (calibration input)
    v_scale: Optional[np.ndarray] = None
    k_inv_scale: Optional[np.ndarray] = None   # float32(1 / scale), what the quantiser multiplies by
    v_inv_scale: Optional[np.ndarray] = None
    note: str = ""

    @property
    def all_requests(self) -> List[Request]:
        return list(self.pre_insert) + [r for b in self.batches for r in b]

    def max_len(self) -> int:
        steps = int(self.decode_tokens.shape[0])
        return max(len(r.tokens) for r in self.all_requests) + steps


class _Builder:
    """Allocates canonical rows and draws tokens with distinct first tokens among siblings."""

    def __init__(self, rng: np.random.Generator, vocab: int):
        self.rng = rng
        self.vocab = vocab
        self.next_row = 0
        # first tokens already used under a given parent segment id
        self.children_first: Dict[int, set] = {}
        self.next_seg = 1   # 0 = root

    def segment(self, parent: int, length: int) -> Tuple[int, np.ndarray, np.ndarray]:
        used = self.children_first.setdefault(parent, set())
        toks = self.rng.integers(0, self.vocab, size=length, dtype=np.int64).astype(np.int32)
        while int(toks[0]) in used:
            toks[0] = int(self.rng.integers(0, self.vocab))
        used.add(int(toks[0]))
        rows = np.arange(self.next_row, self.next_row + length, dtype=np.int64)
        self.next_row += length
        sid = self.next_seg
        self.next_seg += 1
        return sid, toks, rows


def _free_order(rng: np.random.Generator, pool_slots: int, capacity: int) -> np.ndarray:
    return rng.permutation(pool_slots).astype(np.int32)[:capacity]


def _concat(segs) -> Request:
    toks = np.concatenate([s[1] for s in segs]).astype(np.int32)
    rows = np.concatenate([s[2] for s in segs]).astype(np.int64)
    return Request(toks, rows)


def _decode(b: _Builder, n_seq: int, steps: int) -> Tuple[np.ndarray, np.ndarray]:
    toks = b.rng.integers(0, b.vocab, size=(steps, n_seq), dtype=np.int64).astype(np.int32)
    rows = (b.next_row + np.arange(steps * n_seq, dtype=np.int64)).reshape(steps, n_seq)
    b.next_row += steps * n_seq
    return toks, rows


def tiny_f32(seed: int = 1) -> Workload:
    """4 requests, shared 64-token prefix, 16-token suffixes, fp32, 8/8 heads, d 64, 1,024 shuffled slots.

    Nothing is inserted up front: the first request extends all 80 of its tokens and
    the other three reuse its 64-token prefix and extend 16 each."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, 1000)
    shape = Shape(8, 8, 64, "f32", "f32", 1.0 / math.sqrt(64))
    pre = b.segment(0, 64)
    reqs = []
    for i in range(4):
        suf = b.segment(pre[0], 16)
        r = _concat([pre, suf])
        r.tag = f"req{i}"
        reqs.append(r)
    free = _free_order(rng, 1024, 1024)
    dt, dr = _decode(b, 4, 0)
    return Workload("tiny_f32", seed, shape, 1024, free, [], [reqs], True, dt, dr,
                    ValueTable(seed, b.next_row, shape))


def fewshot_bf16(seed: int = 2, n_req: int = 64, prefix_len: int = 1800,
                 suffix_range=(150, 250), decode_steps: int = 1) -> Workload:
    """64 requests sharing a 1,800-token prefix, suffixes U[150, 250]; GQA 32/8, d 128, bf16; 200k slots.

    The prefix is inserted (and its K/V written to the pool) before the batch.
    One decode token per request follows the extend."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, LLAMA3_VOCAB)
    shape = Shape(32, 8, 128, "bf16", "bf16", 1.0 / math.sqrt(128))
    pre = b.segment(0, prefix_len)
    p = Request(pre[1].copy(), pre[2].copy(), "prefix")
    reqs = []
    for i in range(n_req):
        n = int(rng.integers(suffix_range[0], suffix_range[1] + 1))
        r = _concat([pre, b.segment(pre[0], n)])
        r.tag = f"req{i}"
        reqs.append(r)
    free = _free_order(rng, 200_000, 200_000)
    dt, dr = _decode(b, n_req, decode_steps)
    return Workload("fewshot_bf16", seed, shape, 200_000, free, [p], [reqs], True, dt, dr,
                    ValueTable(seed, b.next_row, shape))


def multiturn_bf16(seed: int = 3, n_conv: int = 256, turns: int = 4, turn_range=(64, 512),
                   branch_frac: float = 0.2, batch: int = 32, pool_slots: int = 1_000_000,
                   capacity: int = 262_144) -> Workload:
    """Multi-turn chat: 256 conversations x 4 turns, user/assistant lengths U[64, 512], GQA 32/8, d 128, bf16.

    Turn t's request is the conversation so far plus the new user and assistant runs.
    ``branch_frac`` of the conversations branch once: at a turn tb in {2..turns} they
    rewind to an earlier turn b < tb, keep the user run of turn b, draw a new
    assistant run for it, then a fresh turn; later turns continue from the branch.
    Arrivals are a seeded random interleaving that keeps each conversation's order;
    consecutive arrivals form batches of 32.  The free list holds ``capacity`` of the
    1M pool slots so that LRU eviction fires."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, LLAMA3_VOCAB)
    shape = Shape(32, 8, 128, "bf16", "bf16", 1.0 / math.sqrt(128))
    lo, hi = turn_range
    n_branch = int(math.floor(branch_frac * n_conv))
    branching = set(rng.choice(n_conv, size=n_branch, replace=False).tolist())
    conv_reqs: List[List[Request]] = []
    for c in range(n_conv):
        path = []          # list of segments (sid, toks, rows)
        turn_paths = []    # path after each turn: list of (user_seg, asst_seg)
        tb = int(rng.integers(2, turns + 1)) if c in branching else -1
        reqs = []
        for t in range(1, turns + 1):
            if t == tb:
                bb = int(rng.integers(1, tb))        # rewind to turn bb < tb
                keep = path[: 2 * (bb - 1) + 1]        # u1 a1 ... u_bb
                parent = keep[-1][0]
                a_new = b.segment(parent, int(rng.integers(lo, hi + 1)))
                path = keep + [a_new]
            parent = path[-1][0] if path else 0
            u = b.segment(parent, int(rng.integers(lo, hi + 1)))
            a = b.segment(u[0], int(rng.integers(lo, hi + 1)))
            path = path + [u, a]
            r = _concat(path)
            r.tag = f"conv{c}/turn{t}" + ("/branch" if t == tb else "")
            reqs.append(r)
        conv_reqs.append(reqs)
    order = np.repeat(np.arange(n_conv), turns)
    rng.shuffle(order)
    nxt = [0] * n_conv
    prev = [-1] * n_conv
    arrivals = []
    for c in order.tolist():
        r = conv_reqs[c][nxt[c]]
        r.after = prev[c]
        r.priority = 1 if c % 4 == 0 else 0
        prev[c] = len(arrivals)
        arrivals.append(r)
        nxt[c] += 1
    batches = [arrivals[i:i + batch] for i in range(0, len(arrivals), batch)]
    free = _free_order(rng, pool_slots, capacity)
    dt, dr = _decode(b, len(batches[-1]), 0)
    return Workload("multiturn_bf16", seed, shape, pool_slots, free, [], batches, True, dt, dr,
                    ValueTable(seed, b.next_row, shape),
                    note=f"{n_branch} branching conversations")


def decode_bf16(seed: int = 4, n_seq: int = 512, n_prefix: int = 16, prefix_len: int = 1024,
                ctx_range=(2048, 8192), steps: int = 32, pool_slots: int = 4_194_304) -> Workload:
    """Decode batch: 512 sequences, contexts U[2048, 8192] = one of 16 shared 1,024-token prefixes
    plus a private tail; GQA 32/8, d 128, bf16; 32 decode steps.  The prefixes are inserted first,
    then every sequence is prepared and its K/V written (no extend attention)."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, LLAMA3_VOCAB)
    shape = Shape(32, 8, 128, "bf16", "bf16", 1.0 / math.sqrt(128))
    prefixes = [b.segment(0, prefix_len) for _ in range(n_prefix)]
    pre = [Request(s[1].copy(), s[2].copy(), f"prefix{i}") for i, s in enumerate(prefixes)]
    seqs = []
    for s in range(n_seq):
        L = int(rng.integers(ctx_range[0], ctx_range[1] + 1))
        pfx = prefixes[s % n_prefix]
        r = _concat([pfx, b.segment(pfx[0], L - prefix_len)])
        r.tag = f"seq{s}"
        seqs.append(r)
    free = _free_order(rng, pool_slots, pool_slots)
    dt, dr = _decode(b, n_seq, steps)
    return Workload("decode_bf16", seed, shape, pool_slots, free, pre, [seqs], False, dt, dr,
                    ValueTable(seed, b.next_row, shape))


def longctx_fp8(seed: int = 5, n_req: int = 16, prefix_len: int = 32768, suffix_len: int = 1024,
                steps: int = 64, pool_slots: int = 65_536) -> Workload:
    """Long context: 16 requests share a 32,768-token prefix, 1,024-token suffixes; GQA 64/8, d 128;
    fp8 e4m3 pool with one fp32 scale per (kv-head, K or V); extend, then 64 decode steps."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, LLAMA3_VOCAB)
    shape = Shape(64, 8, 128, "bf16", "fp8_e4m3", 1.0 / math.sqrt(128))
    pfx = b.segment(0, prefix_len)
    pre = [Request(pfx[1].copy(), pfx[2].copy(), "prefix")]
    reqs = []
    for i in range(n_req):
        r = _concat([pfx, b.segment(pfx[0], suffix_len)])
        r.tag = f"req{i}"
        reqs.append(r)
    free = _free_order(rng, pool_slots, pool_slots)
    dt, dr = _decode(b, n_req, steps)
    vt = ValueTable(seed, b.next_row, shape)
    wl = Workload("longctx_fp8", seed, shape, pool_slots, free, pre, [reqs], True, dt, dr, vt)
    wl.k_scale, wl.v_scale = fp8_scales(vt)
    wl.k_inv_scale = (np.float32(1.0) / wl.k_scale).astype(np.float32)
    wl.v_inv_scale = (np.float32(1.0) / wl.v_scale).astype(np.float32)
    return wl


def tot_bf16(seed: int = 6, root_len: int = 1024, branching: int = 4, depth: int = 4, template_len: int = 8,
             thought_range=(96, 224), decode_steps: int = 16, pool_slots: int = 262_144) -> Workload:
    """Tree-of-Thought: a 1,024-token root prompt expanded breadth-first, 4 children per node, 4 levels
    (4 + 16 + 64 + 256 requests); MHA 32/32, d 128 (the LLaMA-7B attention shape), bf16.

    Every node's thought is a step template of 8 tokens shared by all children of one parent,
    then its own U[96, 224] tokens, so siblings share a short run and split it on insert.  The
    request of a node is the root plus the thoughts on its path; each level is one batch, whose
    requests reuse the root and their parent's path (inserted by the level before) and extend
    the template (first sibling only) and the new thought.  The last level decodes 16 tokens."""
    rng = np.random.default_rng(seed)
    b = _Builder(rng, LLAMA3_VOCAB)
    shape = Shape(32, 32, 128, "bf16", "bf16", 1.0 / math.sqrt(128))
    root = b.segment(0, root_len)
    pre = [Request(root[1].copy(), root[2].copy(), "root")]
    lo, hi = thought_range
    frontier = [([root], "n")]
    batches = []
    for level in range(1, depth + 1):
        nxt, reqs = [], []
        for path, name in frontier:
            tpl = b.segment(path[-1][0], template_len)
            for c in range(branching):
                th = b.segment(tpl[0], int(rng.integers(lo, hi + 1)))
                p = path + [tpl, th]
                r = _concat(p)
                r.tag = f"{name}.{c}"
                reqs.append(r)
                nxt.append((p, f"{name}.{c}"))
        batches.append(reqs)
        frontier = nxt
    free = _free_order(rng, pool_slots, pool_slots)
    dt, dr = _decode(b, len(batches[-1]), decode_steps)
    return Workload("tot_bf16", seed, shape, pool_slots, free, pre, batches, True, dt, dr,
                    ValueTable(seed, b.next_row, shape),
                    note=f"{sum(len(x) for x in batches)} requests over {depth} levels")


FP8_E4M3_MAX = 448.0


def fp8_scales(vt: ValueTable) -> Tuple[np.ndarray, np.ndarray]:
    """Per-kv-head calibration: scale = amax / 448 over every value the head holds in the run."""
    out = []
    for tag in (TAG_K, TAG_V):
        amax = np.zeros(vt.shape.hkv, dtype=np.float32)
        n_blocks = (vt.n_rows + BLOCK_ROWS - 1) // BLOCK_ROWS
        for blk in range(n_blocks):
            lo = blk * BLOCK_ROWS
            hi = min(vt.n_rows, lo + BLOCK_ROWS)
            a = vt._gen_block(tag, blk)[: hi - lo].reshape(hi - lo, vt.shape.hkv, vt.shape.d)
            amax = np.maximum(amax, np.abs(a).max(axis=(0, 2)))
        out.append((amax / np.float32(FP8_E4M3_MAX)).astype(np.float32))
    return out[0], out[1]


CONFIGS = {
    "tiny_f32": tiny_f32,
    "fewshot_bf16": fewshot_bf16,
    "multiturn_bf16": multiturn_bf16,
    "decode_bf16": decode_bf16,
    "longctx_fp8": longctx_fp8,
    "tot_bf16": tot_bf16,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)
