"""Host orchestration of the prefix-shared KV path on one GPU.

Holds one radix tree (libpkv's rt_*), the K and V pools ([num_slots, hkv, d] device
tensors) and the per-batch tables, and sequences the library calls of one batch:

    rt_prepare_extend (match / lock / alloc+evict / insert per request, on the host)
    -> H2D copy of req_to_token, lens, qo_indptr, new slots, work plan
    -> pkv_kv_scatter (new tokens' K/V into their slots)
    -> pkv_extend_attention (suffix over reused prefix)
    -> rt_release

and one decode step (rt_decode_step -> H2D -> pkv_kv_scatter -> pkv_decode_attention).
Nothing here computes; it only allocates buffers and passes them to the library.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

from . import (PKV_BF16, PKV_F32, PKV_FP8_E4M3, PKV_NO_SPLIT_PHASE, check, lib, pkv_decode_chunk,
               pkv_decode_first_split, pkv_decode_plan, pkv_decode_shared_rows, pkv_decode_workspace_bytes,
               pkv_extend_plan, pkv_extend_tile, rt_chunk_finish, rt_chunk_prepare, rt_create_policy, rt_decode_step,
               rt_destroy, rt_finish, rt_prepare_extend, rt_prepare_extend_prio, rt_release, rt_serve_round,
               rt_set_eviction_log)

_DT = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8_e4m3": PKV_FP8_E4M3}


@dataclasses.dataclass
class HostBatch:
    """Host tables of one prepared batch (views into the caller's or our own buffers)."""
    n: int
    req_to_token: np.ndarray     # int32 [n, stride]
    prefix_lens: np.ndarray      # int32 [n]
    extend_lens: np.ndarray      # int32 [n]
    qo_indptr: np.ndarray        # int32 [n + 1]
    new_slots: np.ndarray        # int32 [n_new]
    last_nodes: np.ndarray       # int64 [n]
    seq_lens: np.ndarray         # int32 [n]: current length of each sequence (grows with decode)

    @property
    def n_new(self) -> int:
        return int(self.qo_indptr[self.n])


def flatten(token_lists: Sequence[np.ndarray]):
    lens = np.array([len(t) for t in token_lists], dtype=np.int64)
    indptr = np.zeros(len(token_lists) + 1, dtype=np.int64)
    np.cumsum(lens, out=indptr[1:])
    toks = np.concatenate([np.asarray(t, dtype=np.int32) for t in token_lists]) if len(token_lists) else \
        np.zeros(0, dtype=np.int32)
    return np.ascontiguousarray(toks, dtype=np.int32), indptr


def prepare(tree, token_lists, stride: int, r2t: Optional[np.ndarray] = None) -> HostBatch:
    """rt_prepare_extend over a list of token arrays, or over an already flattened
    (tokens, indptr) pair (as `flatten` returns), which saves the concatenation.

    r2t, if given, is the int32 [>= max(n, 1), stride] array the slot rows are written to
    (e.g. a view into a pinned staging buffer); entries past a request's length are then left
    as they were (no kernel reads them), otherwise they are -1."""
    toks, indptr = token_lists if isinstance(token_lists, tuple) else flatten(token_lists)
    n = int(indptr.size - 1)
    if r2t is None:
        r2t = np.full((max(n, 1), stride), -1, dtype=np.int32)
    pl = np.zeros(max(n, 1), dtype=np.int32)
    el = np.zeros(max(n, 1), dtype=np.int32)
    qo = np.zeros(n + 1, dtype=np.int32)
    new = np.empty(max(int(indptr[-1]), 1), dtype=np.int32)
    last = np.full(max(n, 1), -1, dtype=np.int64)
    n_new = rt_prepare_extend(tree, toks, indptr, r2t, pl, el, qo, new, last)
    seq = (indptr[1:] - indptr[:-1]).astype(np.int32)
    return HostBatch(n, r2t[:n], pl[:n], el[:n], qo, new[:n_new], last[:n], seq)


class StagedUpload:
    """Host -> device upload of int32 tables without stalling the launch stream.

    Two pinned host buffers and two device buffers alternate.  With side=True, send() copies
    the current pair on a side stream (default priority) and makes the caller's current
    stream wait for that copy, so a large copy runs while earlier kernels still execute
    instead of between them.  Reuse is safe because the copy into a device buffer first waits
    for a marker recorded on the current stream at the previous send(): everything launched
    before that call, which includes every reader of the buffer's previous contents when
    readers are launched before the next send(), has finished.  Small copies (below
    SIDE_MIN_BYTES, or every copy with side=False) go on the current stream, which orders them
    after those readers by itself: there the side stream's host bookkeeping (~20 µs) costs
    more than the copy.  host() waits for the last copy out of the host buffer."""

    SIDE_MIN_BYTES = 256 << 10

    def __init__(self, torch, device, side: bool = True):
        self.torch = torch
        self.device = device
        self.stream = torch.cuda.Stream(device=device) if side else None
        self.bufs = [dict(host=None, np=None, dev=None, copied=torch.cuda.Event()) for _ in range(2)]
        self.marks = [torch.cuda.Event(), torch.cuda.Event()]
        self.i = 0
        self.seq = 0          # number of send() calls so far
        self.waited = -1      # bufs[i] host side already synchronized for this send

    def host(self, need: int, keep: bool = False) -> np.ndarray:
        """The int32 pinned buffer the next send() copies from, holding at least `need`
        values, once the copy that last read it is done.  keep=True preserves what the buffer
        holds if it has to grow."""
        torch = self.torch
        b = self.bufs[self.i]
        if self.waited != self.seq:
            b["copied"].synchronize()
            self.waited = self.seq
        if b["host"] is None or b["host"].numel() < need:
            old = b["np"]
            b["host"] = torch.empty(max(need * 2, 64), dtype=torch.int32).pin_memory()
            b["np"] = b["host"].numpy()
            if keep and old is not None:
                b["np"][:old.size] = old
        return b["np"]

    def send(self, total: int):
        """Copy the first `total` values of the current host buffer to its device buffer on
        the side stream; returns the device view (int32 [total])."""
        torch = self.torch
        b = self.bufs[self.i]
        if b["host"] is None or b["host"].numel() < total:
            raise ValueError("send() without a large enough host() buffer")
        main = torch.cuda.current_stream(self.device)
        if b["dev"] is None or b["dev"].numel() < total:
            b["dev"] = torch.empty(max(total * 2, 64), dtype=torch.int32, device=self.device)
            if self.stream is not None:
                b["dev"].record_stream(self.stream)
        if self.stream is not None:
            self.marks[self.seq & 1].record(main)    # all work launched so far on the current stream
        if self.stream is None or total * 4 < self.SIDE_MIN_BYTES:
            b["dev"][:total].copy_(b["host"][:total], non_blocking=True)
            b["copied"].record(main)
        else:
            if self.seq > 0:
                # readers of this device buffer's previous contents were launched before the
                # previous send(), whose marker covers them
                self.stream.wait_event(self.marks[(self.seq & 1) ^ 1])
            with torch.cuda.stream(self.stream):
                b["dev"][:total].copy_(b["host"][:total], non_blocking=True)
                b["copied"].record(self.stream)
            main.wait_event(b["copied"])
        self.i ^= 1
        self.seq += 1
        return b["dev"][:total]


class Engine:
    """One radix tree plus its device KV pools."""

    # the two knobs of the library's decode plan (pkv_decode_plan): RESIDENT_WORKGROUPS, the
    # shared-prefix kernel's workgroups the GPU holds at once (two per CU), sets the item span
    # (the launch is costed in rounds of that many workgroups); plans whose items and private
    # tails together need at most PRIVATE_MAX_WORKGROUPS workgroups give the tails to the
    # shared-prefix kernel too
    RESIDENT_WORKGROUPS = 512
    PRIVATE_MAX_WORKGROUPS = 4096
    NO_SPLIT_PHASE = PKV_NO_SPLIT_PHASE

    def __init__(self, num_slots: int, hq: int, hkv: int, d: int, qo_dtype: str, pool_dtype: str,
                 free_order: Optional[np.ndarray] = None, device: str = "cuda", k_scale=None, v_scale=None,
                 k_inv_scale=None, v_inv_scale=None, sm_scale: Optional[float] = None, policy: str = "lru"):
        import torch
        self.torch = torch
        self.num_slots, self.hq, self.hkv, self.d = int(num_slots), hq, hkv, d
        self.qo_code, self.pool_code = _DT[qo_dtype], _DT[pool_dtype]
        self.qo_torch = torch.float32 if qo_dtype == "f32" else torch.bfloat16
        pool_torch = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[pool_dtype]
        self.device = torch.device(device)
        self.tree = rt_create_policy(num_slots, free_order, policy)
        rt_set_eviction_log(self.tree, False)   # nothing here reads it; a serving loop must not grow it
        self.k_pool = torch.zeros((num_slots, hkv, d), dtype=pool_torch, device=self.device)
        self.v_pool = torch.zeros((num_slots, hkv, d), dtype=pool_torch, device=self.device)
        f = lambda a: None if a is None else torch.as_tensor(np.asarray(a, dtype=np.float32), device=self.device)
        self.k_scale, self.v_scale = f(k_scale), f(v_scale)
        self.k_inv_scale, self.v_inv_scale = f(k_inv_scale), f(v_inv_scale)
        self.sm_scale = float(sm_scale if sm_scale is not None else d ** -0.5)
        self.tile = pkv_extend_tile(self.qo_code, self.pool_code, hq, hkv, d)
        self.shared_rows = pkv_decode_shared_rows(self.qo_code, self.pool_code, hq, hkv, d)
        # the step calls below go to the C ABI directly: the pools, scales and shapes are the
        # engine's own (their addresses fixed for its life) and the per-call tensors are its
        # device tables or are checked by shape here; the public binding's per-argument checks
        # cost more host time than a small launch
        ptr = lambda t: 0 if t is None else t.data_ptr()
        self._lib = lib()
        self._pools = (ptr(self.k_pool), ptr(self.v_pool))
        self._scales = (ptr(self.k_scale), ptr(self.v_scale))
        self._inv_scales = (ptr(self.k_inv_scale), ptr(self.v_inv_scale))
        self._cur_stream = torch._C._cuda_getCurrentRawStream
        self._cur_device = torch._C._cuda_getDevice

    def close(self):
        if self.tree is not None:
            rt_destroy(self.tree)
            self.tree = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- host -> device tables ----------------------------------------------------------
    def to_dev(self, a: np.ndarray):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device, non_blocking=False)

    def _uploader(self, name: str, side: bool = True) -> "StagedUpload":
        up = getattr(self, name, None)
        if up is None:
            up = StagedUpload(self.torch, self.device, side)
            setattr(self, name, up)
        return up

    def prepare_staged(self, token_lists, stride: int) -> HostBatch:
        """prepare() whose slot rows are written straight into the pinned buffer the next
        device_tables(staged=True) call uploads (no host copy of the table).  Entries past a
        request's length are unspecified."""
        toks, indptr = token_lists if isinstance(token_lists, tuple) else flatten(token_lists)
        n = max(int(indptr.size - 1), 1)
        up = self._uploader("_tables_up")
        hn = up.host(n * stride + 4 * n + 2 * int(indptr[-1]) + 1024)
        hb = prepare(self.tree, (toks, indptr), stride, r2t=hn[:n * stride].reshape(n, stride))
        hb.staged_in = (up, up.seq)
        return hb

    def device_tables(self, hb: HostBatch, staged: bool = False):
        """Copy one batch's tables (and its extend plan) to the device.

        staged=True packs them into one pinned buffer and copies it on a side stream
        (StagedUpload): the copy overlaps the work already queued, and the current stream
        waits for it before anything launched after this call.  The returned device views
        may be read by work launched on the current stream until the next staged call; a
        batch from prepare_staged already has its slot rows in place."""
        work = pkv_extend_plan(hb.prefix_lens, hb.extend_lens, self.tile).reshape(-1, 2)
        arrays = dict(req_to_token=hb.req_to_token, prefix_lens=hb.prefix_lens, extend_lens=hb.extend_lens,
                      qo_indptr=hb.qo_indptr, new_slots=hb.new_slots, work=work)
        if not staged:
            return {k: self.to_dev(v) for k, v in arrays.items()}
        # all tables in one buffer, the slot rows first, each array 256-byte aligned
        offs, total = {}, 0
        for k, a in arrays.items():
            offs[k] = total
            total += (a.size + 63) // 64 * 64
        total = max(total, 64)
        up = self._uploader("_tables_up")
        inplace = getattr(hb, "staged_in", None) == (up, up.seq)
        hn = up.host(total, keep=inplace)
        for k, a in arrays.items():
            if inplace and k == "req_to_token":
                continue                   # written there by rt_prepare_extend
            hn[offs[k]:offs[k] + a.size] = a.reshape(-1)
        if inplace:
            hb.staged_in = None
        dev = up.send(total)
        return {k: dev[offs[k]:offs[k] + a.size].view(a.shape) for k, a in arrays.items()}

    def upload_decode(self, slots: np.ndarray, seq_lens: np.ndarray, plan=None):
        """One decode step's new slots and sequence lengths on the device (int32 [n] each),
        through a staged upload of their own; valid for work launched on the current stream
        until the next call.  With a host plan (decode_plan(..., upload=False)) it travels in
        the same copy and a third value, the device plan, is returned."""
        n = int(slots.size)
        extra = 0 if plan is None else 2 * n + plan["items"].size
        up = self._uploader("_decode_up", side=False)
        hn = up.host(2 * n + extra)
        hn[:n] = slots
        hn[n:2 * n] = seq_lens
        if plan is None:
            dev = up.send(2 * n)
            return dev[:n], dev[n:2 * n]
        m = plan["items"].size
        hn[2 * n:3 * n] = plan["members"]
        hn[3 * n:4 * n] = plan["skip"]
        hn[4 * n:4 * n + m] = plan["items"].reshape(-1)
        dev = up.send(4 * n + m)
        first = self.first_split(plan["skip"], seq_lens, plan["chunk"])
        return dev[:n], dev[n:2 * n], dict(members=dev[2 * n:3 * n], skip=dev[3 * n:4 * n],
                                           items=dev[4 * n:4 * n + m].view(-1, 4), chunk=plan["chunk"],
                                           first_split=first)

    @staticmethod
    def first_split(skip: np.ndarray, seq_lens: np.ndarray, chunk: int) -> int:
        """The first chunk the split phase must launch for a plan's skip at the current
        lengths (pkv_decode_first_split), or NO_SPLIT_PHASE."""
        return pkv_decode_first_split(skip, seq_lens, chunk)

    # -- steps ---------------------------------------------------------------------------
    def prepare(self, token_lists, stride: int) -> HostBatch:
        return prepare(self.tree, token_lists, stride)

    def _stream(self):
        return self._cur_stream(self._cur_device())

    def _rows(self, t, n, what):
        """A contiguous device tensor of n rows of [hkv, d]."""
        if t.shape != (n, self.hkv, self.d) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{what}: expected a contiguous device tensor [{n}, {self.hkv}, {self.d}]")
        return t.data_ptr()

    def _src_code(self, t):
        if t.dtype == self.torch.bfloat16:
            return PKV_BF16
        if t.dtype == self.torch.float32:
            return PKV_F32
        raise TypeError(f"unsupported source dtype {t.dtype}")

    def scatter(self, slots_dev, k_new, v_new):
        n = int(slots_dev.shape[0])
        if slots_dev.dtype != self.torch.int32 or not slots_dev.is_contiguous() or v_new.dtype != k_new.dtype:
            raise ValueError("scatter: slots must be contiguous int32, k and v of one dtype")
        check(self._lib.pkv_kv_scatter(self._rows(k_new, n, "k_new"), self._rows(v_new, n, "v_new"),
                                       self._src_code(k_new), slots_dev.data_ptr(), n, *self._pools,
                                       self.pool_code, self.num_slots, self.hkv, self.d, *self._inv_scales,
                                       self._stream()))

    def extend(self, dt, q, o=None):
        if o is None:
            o = self.torch.empty_like(q)
        n = int(q.shape[0])
        if q.shape != (n, self.hq, self.d) or o.shape != q.shape or q.dtype != self.qo_torch \
                or o.dtype != q.dtype or not (q.is_contiguous() and o.is_contiguous()):
            raise ValueError("extend: q and o must be contiguous [rows, hq, d] in the engine's dtype")
        r2t = dt["req_to_token"]
        work = dt["work"]
        if r2t.dtype != self.torch.int32 or work.dtype != self.torch.int32:
            raise ValueError("extend: tables must be int32 (Engine.device_tables)")
        check(self._lib.pkv_extend_attention(q.data_ptr(), o.data_ptr(), self.qo_code, *self._pools, self.pool_code,
                                             self.num_slots, *self._scales, r2t.data_ptr(), r2t.shape[1],
                                             dt["prefix_lens"].data_ptr(), dt["extend_lens"].data_ptr(),
                                             dt["qo_indptr"].data_ptr(), dt["prefix_lens"].shape[0],
                                             work.data_ptr(), work.shape[0], self.hq, self.hkv, self.d,
                                             self.sm_scale, self._stream()))
        return o

    def append_slots(self, r2t_dev, seq_lens_dev, slots_dev):
        """Device side of a decode step's table emit (pkv_append_slots) on the engine's tables."""
        b = int(slots_dev.shape[0])
        if seq_lens_dev.shape != (b,) or r2t_dev.dim() != 2 or r2t_dev.shape[0] < b \
                or r2t_dev.dtype != self.torch.int32:
            raise ValueError("append_slots: shape mismatch")
        check(self._lib.pkv_append_slots(r2t_dev.data_ptr(), r2t_dev.shape[1], seq_lens_dev.data_ptr(),
                                         slots_dev.data_ptr(), b, self._stream()))

    def release(self, hb: HostBatch):
        rt_release(self.tree, hb.last_nodes)

    def decode_alloc(self, hb: HostBatch) -> np.ndarray:
        out = np.empty(hb.n, dtype=np.int32)
        rt_decode_step(self.tree, hb.req_to_token, hb.seq_lens, out)
        return out

    def decode_workspace(self, batch: int, max_seq_len: int, chunk: int = 0):
        chunk = chunk or pkv_decode_chunk(batch, self.hkv, max_seq_len)
        nbytes = pkv_decode_workspace_bytes(batch, self.hq, self.d, max_seq_len, chunk)
        return self.torch.empty(nbytes // 4 + 1, dtype=self.torch.float32, device=self.device), chunk

    def decode_plan(self, req_to_token: np.ndarray, seq_lens: np.ndarray, chunk: int, upload: bool = True):
        """The library's shared-prefix plan of a decode batch (pkv_decode_plan over the host slot
        rows and current lengths), or None when no chunk is shared or the shape has no
        shared-prefix kernel.  Computed once, it serves every later decode step of the same
        sequences (new tokens are private, so the shared chunks do not change; a chunk a
        sequence grows into is left to the split phase, which decode() launches from the
        first split at that step's lengths).  upload=True: a dict of device int32 views
        (members, skip, items) valid for work launched before the next call, plus the host
        skip; upload=False: the host arrays, for upload_decode to send with a step's slots."""
        rows = self.shared_rows
        if rows <= 0:
            return None
        # the rows come from this engine's tree (its locks keep them)
        plan = pkv_decode_plan(req_to_token, seq_lens, chunk, rows, self.hkv, self.RESIDENT_WORKGROUPS,
                               self.PRIVATE_MAX_WORKGROUPS)
        if plan is None:
            return None
        members, skip, items, first = plan
        if not upload:
            return dict(members=members, skip=skip, items=items, chunk=int(chunk), first_split=first)
        b, n = members.size, items.size
        up = self._uploader("_plan_up", side=False)
        hn = up.host(2 * b + n)
        hn[:b] = members
        hn[b:2 * b] = skip
        hn[2 * b:2 * b + n] = items.reshape(-1)
        dev = up.send(2 * b + n)
        return dict(members=dev[:b], skip=dev[b:2 * b], items=dev[2 * b:2 * b + n].view(-1, 4), chunk=int(chunk),
                    first_split=first, skip_host=skip.copy())

    def decode(self, q, r2t_dev, seq_lens_dev, max_seq_len: int, workspace, chunk: int, o=None, plan=None,
               seq_lens_host=None):
        """One decode step; with a plan from decode_plan (same chunk), the shared chunks are
        read once per group of sequences.  seq_lens_host (this step's lengths) sets the split
        phase's first chunk for a plan made at an earlier step; without it the plan's own
        first_split (right at the step it was made for) is used."""
        if o is None:
            o = self.torch.empty_like(q)
        b = int(q.shape[0])
        if q.shape != (b, self.hq, self.d) or o.shape != q.shape or q.dtype != self.qo_torch \
                or o.dtype != q.dtype or not (q.is_contiguous() and o.is_contiguous()) \
                or seq_lens_dev.shape != (b,) or r2t_dev.dim() != 2 or r2t_dev.shape[0] < b \
                or r2t_dev.dtype != self.torch.int32 or seq_lens_dev.dtype != self.torch.int32:
            raise ValueError("decode: shape mismatch")
        head = (q.data_ptr(), o.data_ptr(), self.qo_code, *self._pools, self.pool_code, self.num_slots,
                *self._scales, r2t_dev.data_ptr(), r2t_dev.shape[1], seq_lens_dev.data_ptr(), b, int(max_seq_len),
                self.hq, self.hkv, self.d, self.sm_scale, int(chunk))
        ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), self._stream())
        if plan is not None:
            if plan["chunk"] != chunk or plan["members"].shape != (b,):
                raise ValueError("decode: the plan was made for another chunk or batch")
            items = plan["items"]
            first = plan["first_split"]
            if seq_lens_host is not None and plan.get("skip_host") is not None:
                first = pkv_decode_first_split(plan["skip_host"], seq_lens_host, chunk)
            check(self._lib.pkv_decode_attention_shared(*head, plan["members"].data_ptr(), plan["skip"].data_ptr(),
                                                        items.data_ptr(), items.shape[0], first, *ws))
        else:
            check(self._lib.pkv_decode_attention(*head, *ws))
        return o

    def finish(self, hb: HostBatch, full_token_lists, prompt_lens):
        toks, indptr = full_token_lists if isinstance(full_token_lists, tuple) else flatten(full_token_lists)
        return rt_finish(self.tree, toks, indptr, hb.req_to_token, prompt_lens, hb.last_nodes)


def run_workload_host(wl, release_last_batch: bool = True, policy: str = "lru"):
    """Drive a workload's host steps through the library's tree (no device work).

    Returns (batches, decode slots per step, eviction log, free list, evictable, protected, dump)."""
    from . import (rt_copy_free_list, rt_dump, rt_evictable_size, rt_protected_size, rt_take_eviction_log)
    tree = rt_create_policy(wl.pool_slots, wl.free_order, policy)
    try:
        stride = wl.max_len()
        for r in wl.pre_insert:
            hb = prepare(tree, [r.tokens], stride)
            rt_release(tree, hb.last_nodes)
        batches = []
        for bi, batch in enumerate(wl.batches):
            hb = prepare(tree, [r.tokens for r in batch], stride)
            batches.append(hb)
            if bi < len(wl.batches) - 1:
                rt_release(tree, hb.last_nodes)
        steps = int(wl.decode_tokens.shape[0])
        last = batches[-1]
        dec = []
        for _ in range(steps):
            out = np.empty(last.n, dtype=np.int32)
            rt_decode_step(tree, last.req_to_token, last.seq_lens, out)
            dec.append(out.tolist())
        if steps:
            full = [np.concatenate([r.tokens, wl.decode_tokens[:, i]]) for i, r in enumerate(wl.batches[-1])]
            toks, indptr = flatten(full)
            rt_finish(tree, toks, indptr, last.req_to_token, [len(r.tokens) for r in wl.batches[-1]],
                      last.last_nodes)
        elif release_last_batch:
            rt_release(tree, last.last_nodes)
        return (batches, dec, rt_take_eviction_log(tree), rt_copy_free_list(tree).tolist(), rt_evictable_size(tree),
                rt_protected_size(tree), rt_dump(tree))
    finally:
        rt_destroy(tree)


def prepare_prio(tree, token_lists: Sequence[np.ndarray], stride: int, priorities=None) -> HostBatch:
    """prepare() whose inserts carry one priority per request."""
    toks, indptr = flatten(token_lists)
    n = len(token_lists)
    r2t = np.full((max(n, 1), stride), -1, dtype=np.int32)
    pl = np.zeros(max(n, 1), dtype=np.int32)
    el = np.zeros(max(n, 1), dtype=np.int32)
    qo = np.zeros(n + 1, dtype=np.int32)
    new = np.empty(max(int(indptr[-1]), 1), dtype=np.int32)
    last = np.full(max(n, 1), -1, dtype=np.int64)
    n_new = rt_prepare_extend_prio(tree, toks, indptr, priorities, r2t, pl, el, qo, new, last)
    seq = (indptr[1:] - indptr[:-1]).astype(np.int32)
    return HostBatch(n, r2t[:n], pl[:n], el[:n], qo, new[:n_new], last[:n], seq)


def serve(tree, token_lists: Sequence[np.ndarray], after: Sequence[int], order: str, batch: int, window: int,
          stride: int, priorities=None, on_batch=None):
    """Cache-aware serve loop over a fixed arrival order, one batch per round: the library
    picks each round (rt_serve_round: the `window` oldest unscheduled requests, those whose
    `after` request ran in an earlier round, in arrival order for "fcfs" or longest cached
    prefix first for "lpm"); the batch is prepared, handed to on_batch(pick, host_batch) for
    its device work, and released.  Returns [(pick, host_batch)] in round order."""
    toks, indptr = flatten(token_lists)
    scheduled = np.zeros(len(token_lists), dtype=np.uint8)
    out = []
    while True:
        pick = rt_serve_round(tree, toks, indptr, after, scheduled, window, order, batch).tolist()
        if not pick:
            return out
        hb = prepare_prio(tree, [token_lists[i] for i in pick], stride,
                          None if priorities is None else [priorities[i] for i in pick])
        if on_batch is not None:
            on_batch(pick, hb)
        rt_release(tree, hb.last_nodes)
        scheduled[pick] = 1
        out.append((pick, hb))


def chunked_prefill(tree, token_lists: Sequence[np.ndarray], budget: int, stride: int, on_launch=None):
    """Prefill one batch in launches of at most `budget` new tokens: the library cuts and
    prepares each launch (rt_chunk_prepare: requests in order, a request cut by the budget
    continues in the next launch, its earlier chunks reused through the tree and kept locked
    until the continuation is prepared); on_launch(reqs, ends, host_batch) runs the launch's
    device work; rt_chunk_finish then unlocks the requests that reached their end.
    Returns [(reqs, ends, host_batch)]."""
    if budget < 1:
        raise ValueError("chunk budget must be positive")
    n = len(token_lists)
    toks, indptr = flatten(token_lists)
    done = np.full(n, -1, dtype=np.int64)
    held = np.full(n, -1, dtype=np.int64)
    out = []
    head = 0
    while head < n:
        r2t = np.full((n - head, stride), -1, dtype=np.int32)
        reqs, ends, pl, el, qo, new = rt_chunk_prepare(tree, toks, indptr, done, held, head, budget, r2t)
        k = int(reqs.size)
        hb = HostBatch(k, r2t[:k], pl, el, qo, new, held[reqs].copy(), ends.astype(np.int32))
        if on_launch is not None:
            on_launch(reqs.tolist(), ends.tolist(), hb)
        head = rt_chunk_finish(tree, indptr, reqs, done, held, head)
        out.append((reqs.tolist(), ends.tolist(), hb))
    return out
