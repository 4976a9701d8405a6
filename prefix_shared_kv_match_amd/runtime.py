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

from . import (PKV_BF16, PKV_F32, PKV_FP8_E4M3, pkv_decode_attention, pkv_decode_chunk,
               pkv_decode_workspace_bytes, pkv_extend_attention, pkv_extend_plan, pkv_extend_tile, pkv_kv_scatter,
               rt_create, rt_decode_step, rt_destroy, rt_finish, rt_prepare_extend, rt_release)

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


def prepare(tree, token_lists: Sequence[np.ndarray], stride: int) -> HostBatch:
    toks, indptr = flatten(token_lists)
    n = len(token_lists)
    r2t = np.full((max(n, 1), stride), -1, dtype=np.int32)
    pl = np.zeros(max(n, 1), dtype=np.int32)
    el = np.zeros(max(n, 1), dtype=np.int32)
    qo = np.zeros(n + 1, dtype=np.int32)
    new = np.empty(max(int(indptr[-1]), 1), dtype=np.int32)
    last = np.full(max(n, 1), -1, dtype=np.int64)
    n_new = rt_prepare_extend(tree, toks, indptr, r2t, pl, el, qo, new, last)
    seq = (indptr[1:] - indptr[:-1]).astype(np.int32)
    return HostBatch(n, r2t[:n], pl[:n], el[:n], qo, new[:n_new], last[:n], seq)


class Engine:
    """One radix tree plus its device KV pools."""

    def __init__(self, num_slots: int, hq: int, hkv: int, d: int, qo_dtype: str, pool_dtype: str,
                 free_order: Optional[np.ndarray] = None, device: str = "cuda", k_scale=None, v_scale=None,
                 k_inv_scale=None, v_inv_scale=None, sm_scale: Optional[float] = None):
        import torch
        self.torch = torch
        self.num_slots, self.hq, self.hkv, self.d = int(num_slots), hq, hkv, d
        self.qo_code, self.pool_code = _DT[qo_dtype], _DT[pool_dtype]
        self.qo_torch = torch.float32 if qo_dtype == "f32" else torch.bfloat16
        pool_torch = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[pool_dtype]
        self.device = torch.device(device)
        self.tree = rt_create(num_slots, free_order)
        self.k_pool = torch.zeros((num_slots, hkv, d), dtype=pool_torch, device=self.device)
        self.v_pool = torch.zeros((num_slots, hkv, d), dtype=pool_torch, device=self.device)
        f = lambda a: None if a is None else torch.as_tensor(np.asarray(a, dtype=np.float32), device=self.device)
        self.k_scale, self.v_scale = f(k_scale), f(v_scale)
        self.k_inv_scale, self.v_inv_scale = f(k_inv_scale), f(v_inv_scale)
        self.sm_scale = float(sm_scale if sm_scale is not None else d ** -0.5)
        self.tile = pkv_extend_tile(self.qo_code, self.pool_code, hq, hkv, d)

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

    def device_tables(self, hb: HostBatch, staged: bool = False):
        """Copy one batch's tables (and its extend plan) to the device.

        staged=True copies through two alternating pinned host buffers with asynchronous
        copies on the current stream, so the host can prepare the next batch while the GPU
        still works on this one; the returned device tensors are reused by the next staged
        call (stream order keeps that safe)."""
        work = pkv_extend_plan(hb.prefix_lens, hb.extend_lens, self.tile).reshape(-1, 2)
        arrays = dict(req_to_token=hb.req_to_token, prefix_lens=hb.prefix_lens, extend_lens=hb.extend_lens,
                      qo_indptr=hb.qo_indptr, new_slots=hb.new_slots, work=work)
        if not staged:
            return {k: self.to_dev(v) for k, v in arrays.items()}
        torch = self.torch
        if not hasattr(self, "_stage"):
            self._stage = [dict(host={}, event=torch.cuda.Event()) for _ in range(2)]
            self._stage_i = 0
            self._dev_tables = {}
        st = self._stage[self._stage_i]
        self._stage_i ^= 1
        st["event"].synchronize()          # the copies that last read these pinned buffers are done
        out = {}
        for k, a in arrays.items():
            a = np.ascontiguousarray(a)
            h = st["host"].get(k)
            if h is None or h.numel() < a.size:
                h = torch.empty(max(a.size, 1) * 2, dtype=torch.int32).pin_memory()
                st["host"][k] = h
            d = self._dev_tables.get(k)
            if d is None or d.numel() < a.size:
                d = torch.empty(max(a.size, 1) * 2, dtype=torch.int32, device=self.device)
                self._dev_tables[k] = d
            h.numpy()[:a.size] = a.reshape(-1)
            dv = d[:a.size]
            dv.copy_(h[:a.size], non_blocking=True)
            out[k] = dv.view(a.shape)
        st["event"].record()
        return out

    # -- steps ---------------------------------------------------------------------------
    def prepare(self, token_lists, stride: int) -> HostBatch:
        return prepare(self.tree, token_lists, stride)

    def scatter(self, slots_dev, k_new, v_new):
        pkv_kv_scatter(k_new, v_new, slots_dev, self.k_pool, self.v_pool, self.k_inv_scale, self.v_inv_scale)

    def extend(self, dt, q, o=None):
        if o is None:
            o = self.torch.empty_like(q)
        pkv_extend_attention(q, o, self.k_pool, self.v_pool, dt["req_to_token"], dt["prefix_lens"],
                             dt["extend_lens"], dt["qo_indptr"], dt["work"], self.sm_scale, self.k_scale,
                             self.v_scale)
        return o

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

    def decode(self, q, r2t_dev, seq_lens_dev, max_seq_len: int, workspace, chunk: int, o=None):
        if o is None:
            o = self.torch.empty_like(q)
        pkv_decode_attention(q, o, self.k_pool, self.v_pool, r2t_dev, seq_lens_dev, max_seq_len, self.sm_scale,
                             workspace, chunk, self.k_scale, self.v_scale)
        return o

    def finish(self, hb: HostBatch, full_token_lists, prompt_lens):
        toks, indptr = flatten(full_token_lists)
        return rt_finish(self.tree, toks, indptr, hb.req_to_token, prompt_lens, hb.last_nodes)


def run_workload_host(wl, release_last_batch: bool = True):
    """Drive a workload's host steps through the library's tree (no device work).

    Returns (batches, decode slots per step, eviction log, free list, evictable, protected, dump)."""
    from . import (rt_copy_free_list, rt_dump, rt_evictable_size, rt_protected_size, rt_take_eviction_log)
    tree = rt_create(wl.pool_slots, wl.free_order)
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
