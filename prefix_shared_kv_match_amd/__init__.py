"""prefix_shared_kv_match_amd: prefix-shared KV reuse (radix tree + gathered attention) for MI355X.

Python binding of libpkv.so.  Every function here has the name of the C entry point it
calls (include/pkv.h) and only marshals arguments: host arrays as numpy, device buffers
as torch tensors on a ROCm device.  Every step of the path runs in the library; if the
library is missing, importing the binding functions raises.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from ._capi import (PKV_BF16, PKV_DECODE_STATIC_SCRATCH_BYTES, PKV_F32, PKV_FP8_E4M3, PKV_NO_SPLIT_PHASE, PkvError,
                    check, lib)

__all__ = [
    "PKV_F32", "PKV_BF16", "PKV_FP8_E4M3", "PkvError", "lib",
    "RT_POLICIES", "rt_create", "rt_create_policy", "rt_destroy", "rt_match_prefix", "rt_insert",
    "rt_insert_priority", "rt_peek_prefix", "rt_schedule_longest_prefix", "rt_dump_stats", "rt_prepare_extend_prio",
    "rt_inc_lock_ref", "rt_dec_lock_ref",
    "rt_evict", "rt_alloc", "rt_free", "rt_take_eviction_log", "rt_set_eviction_log", "rt_evictable_size",
    "rt_protected_size",
    "rt_free_size", "rt_clock", "rt_copy_free_list", "rt_dump", "rt_prepare_extend", "rt_release",
    "rt_decode_step", "rt_finish", "rt_serve_round", "rt_chunk_launch", "rt_chunk_prepare", "rt_chunk_finish",
    "pkv_kv_scatter", "pkv_append_slots", "pkv_extend_tile", "pkv_extend_plan",
    "pkv_extend_attention", "pkv_decode_chunk", "pkv_decode_workspace_bytes", "pkv_decode_attention",
    "pkv_decode_shared_rows", "pkv_decode_shared_plan", "pkv_decode_attention_shared",
    "pkv_decode_attention_static", "PKV_DECODE_STATIC_SCRATCH_BYTES",
]

import ctypes as C


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: Optional[np.ndarray]):
    # the buffer address as an int (ctypes passes it for a void* argument); the caller keeps
    # the array alive for the duration of the call
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------------------------------
# radix tree (host)
# ------------------------------------------------------------------------------------------

def rt_create(num_slots: int, free_order: Optional[Sequence[int]] = None) -> C.c_void_p:
    h = C.c_void_p()
    if free_order is None:
        check(lib().rt_create(int(num_slots), None, int(num_slots), C.byref(h)))
    else:
        fo = _i32(free_order)
        check(lib().rt_create(int(num_slots), _ptr(fo), fo.size, C.byref(h)))
    return h


# rt_policy codes of include/pkv.h, by name
RT_POLICIES = {"lru": 0, "lfu": 1, "slru": 2, "fifo": 3, "mru": 4, "filo": 5, "priority": 6}


def rt_create_policy(num_slots: int, free_order: Optional[Sequence[int]] = None, policy="lru") -> C.c_void_p:
    code = RT_POLICIES[policy] if isinstance(policy, str) else int(policy)
    h = C.c_void_p()
    if free_order is None:
        check(lib().rt_create_policy(int(num_slots), None, int(num_slots), code, C.byref(h)))
    else:
        fo = _i32(free_order)
        check(lib().rt_create_policy(int(num_slots), _ptr(fo), fo.size, code, C.byref(h)))
    return h


def rt_destroy(t) -> None:
    lib().rt_destroy(t)


def rt_match_prefix(t, key) -> Tuple[int, np.ndarray, int]:
    key = _i32(key)
    out = np.empty(max(key.size, 1), dtype=np.int32)
    last = C.c_int64()
    m = check(lib().rt_match_prefix(t, _ptr(key), key.size, _ptr(out), C.byref(last)))
    return int(m), out[:m].copy(), int(last.value)


def rt_insert(t, key, slots) -> Tuple[int, int]:
    key, slots = _i32(key), _i32(slots)
    if key.size != slots.size:
        raise ValueError("key and slots differ in length")
    last = C.c_int64()
    m = check(lib().rt_insert(t, _ptr(key), _ptr(slots), key.size, C.byref(last)))
    return int(m), int(last.value)


def rt_insert_priority(t, key, slots, priority: int) -> Tuple[int, int]:
    key, slots = _i32(key), _i32(slots)
    if key.size != slots.size:
        raise ValueError("key and slots differ in length")
    last = C.c_int64()
    m = check(lib().rt_insert_priority(t, _ptr(key), _ptr(slots), key.size, int(priority), C.byref(last)))
    return int(m), int(last.value)


def rt_peek_prefix(t, key) -> int:
    key = _i32(key)
    return int(check(lib().rt_peek_prefix(t, _ptr(key), key.size)))


def rt_schedule_longest_prefix(t, tokens: np.ndarray, tok_indptr: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(order, match_lens): waiting requests by descending cached-prefix length, ties in index order."""
    tokens = _i32(tokens)
    tok_indptr = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    n = int(tok_indptr.size - 1)
    order = np.empty(max(n, 1), dtype=np.int32)
    lens = np.empty(max(n, 1), dtype=np.int64)
    check(lib().rt_schedule_longest_prefix(t, n, _ptr(tokens), _ptr(tok_indptr), _ptr(order), _ptr(lens)))
    return order[:n], lens[:n]


def rt_dump_stats(t):
    """Live non-root nodes as (id, hit count, creation clock, priority), by id."""
    need = check(lib().rt_dump_stats(t, None, 0))
    buf = np.empty(max(need, 1), dtype=np.int64)
    check(lib().rt_dump_stats(t, _ptr(buf), need))
    return [tuple(int(x) for x in buf[k:k + 4]) for k in range(0, need, 4)]


def rt_inc_lock_ref(t, node: int) -> None:
    check(lib().rt_inc_lock_ref(t, int(node)))


def rt_dec_lock_ref(t, node: int) -> None:
    check(lib().rt_dec_lock_ref(t, int(node)))


def rt_evict(t, num_tokens: int) -> int:
    return int(check(lib().rt_evict(t, int(num_tokens))))


def rt_alloc(t, n: int) -> np.ndarray:
    out = np.empty(max(int(n), 1), dtype=np.int32)
    check(lib().rt_alloc(t, int(n), _ptr(out)))
    return out[:n]


def rt_free(t, slots) -> None:
    s = _i32(slots)
    check(lib().rt_free(t, _ptr(s), s.size))


def rt_set_eviction_log(t, enabled: bool) -> None:
    check(lib().rt_set_eviction_log(t, 1 if enabled else 0))


def rt_take_eviction_log(t) -> List[Tuple[int, List[int]]]:
    nn, ns = C.c_int64(), C.c_int64()
    check(lib().rt_eviction_log_size(t, C.byref(nn), C.byref(ns)))
    ids = np.empty(max(nn.value, 1), dtype=np.int64)
    lens = np.empty(max(nn.value, 1), dtype=np.int64)
    slots = np.empty(max(ns.value, 1), dtype=np.int32)
    check(lib().rt_take_eviction_log(t, _ptr(ids), _ptr(lens), nn.value, _ptr(slots), ns.value))
    out, k = [], 0
    for i in range(nn.value):
        out.append((int(ids[i]), slots[k:k + lens[i]].tolist()))
        k += int(lens[i])
    return out


def rt_evictable_size(t) -> int:
    return int(check(lib().rt_evictable_size(t)))


def rt_protected_size(t) -> int:
    return int(check(lib().rt_protected_size(t)))


def rt_free_size(t) -> int:
    return int(check(lib().rt_free_size(t)))


def rt_clock(t) -> int:
    return int(check(lib().rt_clock(t)))


def rt_copy_free_list(t) -> np.ndarray:
    n = rt_free_size(t)
    out = np.empty(max(n, 1), dtype=np.int32)
    check(lib().rt_copy_free_list(t, _ptr(out), n))
    return out[:n]


def rt_dump(t):
    """Live non-root nodes as (id, parent, lock_ref, last_access, key tuple, slots tuple), by id."""
    need = check(lib().rt_dump(t, None, 0))
    buf = np.empty(max(need, 1), dtype=np.int64)
    check(lib().rt_dump(t, _ptr(buf), need))
    out, k = [], 0
    while k < need:
        nid, par, lock, last, n = (int(x) for x in buf[k:k + 5])
        key = tuple(int(x) for x in buf[k + 5:k + 5 + n])
        val = tuple(int(x) for x in buf[k + 5 + n:k + 5 + 2 * n])
        out.append((nid, par, lock, last, key, val))
        k += 5 + 2 * n
    return out


def rt_prepare_extend(t, tokens: np.ndarray, tok_indptr: np.ndarray, req_to_token: np.ndarray,
                      prefix_lens: np.ndarray, extend_lens: np.ndarray, qo_indptr: np.ndarray,
                      new_slots: np.ndarray, out_last: np.ndarray) -> int:
    """Fills the caller's host arrays (see include/pkv.h); returns the number of new tokens."""
    n = int(tok_indptr.size - 1)
    for a, dt in ((tokens, np.int32), (tok_indptr, np.int64), (req_to_token, np.int32), (prefix_lens, np.int32),
                  (extend_lens, np.int32), (qo_indptr, np.int32), (new_slots, np.int32), (out_last, np.int64)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise TypeError("rt_prepare_extend: host arrays must be C-contiguous with the documented dtypes")
    if req_to_token.ndim != 2 or req_to_token.shape[0] < n or prefix_lens.size < n or extend_lens.size < n \
            or qo_indptr.size < n + 1 or out_last.size < n:
        raise ValueError("rt_prepare_extend: output arrays too small")
    return int(check(lib().rt_prepare_extend(t, n, _ptr(tokens), _ptr(tok_indptr), _ptr(req_to_token),
                                             req_to_token.shape[1], _ptr(prefix_lens), _ptr(extend_lens),
                                             _ptr(qo_indptr), _ptr(new_slots), new_slots.size, _ptr(out_last))))


def rt_prepare_extend_prio(t, tokens: np.ndarray, tok_indptr: np.ndarray, priorities, req_to_token: np.ndarray,
                           prefix_lens: np.ndarray, extend_lens: np.ndarray, qo_indptr: np.ndarray,
                           new_slots: np.ndarray, out_last: np.ndarray) -> int:
    """rt_prepare_extend whose inserts carry one priority per request (None = all 0)."""
    n = int(tok_indptr.size - 1)
    for a, dt in ((tokens, np.int32), (tok_indptr, np.int64), (req_to_token, np.int32), (prefix_lens, np.int32),
                  (extend_lens, np.int32), (qo_indptr, np.int32), (new_slots, np.int32), (out_last, np.int64)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise TypeError("rt_prepare_extend_prio: host arrays must be C-contiguous with the documented dtypes")
    if req_to_token.ndim != 2 or req_to_token.shape[0] < n or prefix_lens.size < n or extend_lens.size < n \
            or qo_indptr.size < n + 1 or out_last.size < n:
        raise ValueError("rt_prepare_extend_prio: output arrays too small")
    pr = None if priorities is None else _i32(priorities)
    if pr is not None and pr.size < n:
        raise ValueError("rt_prepare_extend_prio: one priority per request")
    return int(check(lib().rt_prepare_extend_prio(t, n, _ptr(tokens), _ptr(tok_indptr), _ptr(pr), _ptr(req_to_token),
                                                  req_to_token.shape[1], _ptr(prefix_lens), _ptr(extend_lens),
                                                  _ptr(qo_indptr), _ptr(new_slots), new_slots.size,
                                                  _ptr(out_last))))


def rt_release(t, nodes) -> None:
    a = np.ascontiguousarray(nodes, dtype=np.int64)
    check(lib().rt_release(t, _ptr(a), a.size))


def rt_decode_step(t, req_to_token: np.ndarray, seq_lens: np.ndarray, out_slots: np.ndarray) -> int:
    b = int(seq_lens.size)
    if req_to_token.dtype != np.int32 or seq_lens.dtype != np.int32 or out_slots.dtype != np.int32 \
            or out_slots.size < b or req_to_token.shape[0] < b:
        raise TypeError("rt_decode_step: bad host arrays")
    return int(check(lib().rt_decode_step(t, b, _ptr(req_to_token), req_to_token.shape[1], _ptr(seq_lens),
                                          _ptr(out_slots))))


def rt_finish(t, tokens: np.ndarray, tok_indptr: np.ndarray, req_to_token: np.ndarray, prompt_lens,
              prompt_last) -> np.ndarray:
    n = int(tok_indptr.size - 1)
    pl = _i32(prompt_lens)
    last = np.ascontiguousarray(prompt_last, dtype=np.int64)
    ends = np.empty(max(n, 1), dtype=np.int64)
    toks = _i32(tokens)
    ip = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    check(lib().rt_finish(t, n, _ptr(toks), _ptr(ip), _ptr(req_to_token), req_to_token.shape[1], _ptr(pl),
                          _ptr(last), _ptr(ends)))
    return ends[:n]


def rt_chunk_launch(t, tokens: np.ndarray, tok_indptr: np.ndarray, done, head: int, budget: int):
    """One chunked-prefill launch from request `head` on: (requests taken, end position of each
    one's chunk).  done[r] >= 0: request r is under way with done[r] tokens prefilled; -1: not
    started (its cached prefix is skipped)."""
    ip = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    n = int(ip.size - 1)
    dn = np.ascontiguousarray(done, dtype=np.int64)
    if dn.size != n:
        raise ValueError("rt_chunk_launch: done must hold one entry per request")
    toks = _i32(tokens)
    reqs = np.empty(max(n - int(head), 1), dtype=np.int32)
    ends = np.empty(max(n - int(head), 1), dtype=np.int64)
    k = int(check(lib().rt_chunk_launch(t, n, _ptr(toks), _ptr(ip), _ptr(dn), int(head), int(budget), _ptr(reqs),
                                        _ptr(ends))))
    return reqs[:k], ends[:k]


def rt_chunk_prepare(t, tokens: np.ndarray, tok_indptr: np.ndarray, done: np.ndarray, held: np.ndarray, head: int,
                     budget: int, req_to_token: np.ndarray):
    """One chunked-prefill launch: (requests taken, chunk ends, prefix_lens, extend_lens,
    qo_indptr, new_slots) for the taken requests, their rows written into req_to_token
    [>= taken, stride]; done / held (int64 [num_reqs], -1 before the first launch) are
    updated in place."""
    ip = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    n = int(ip.size - 1)
    if done.dtype != np.int64 or held.dtype != np.int64 or done.size != n or held.size != n \
            or not done.flags.c_contiguous or not held.flags.c_contiguous:
        raise ValueError("rt_chunk_prepare: done and held must be contiguous int64 [num_reqs]")
    if req_to_token.dtype != np.int32 or req_to_token.ndim != 2 or not req_to_token.flags.c_contiguous:
        raise ValueError("rt_chunk_prepare: req_to_token must be a contiguous int32 [rows, stride] array")
    toks = _i32(tokens)
    cap = max(n - int(head), 1)
    if req_to_token.shape[0] < cap:
        raise ValueError("rt_chunk_prepare: req_to_token needs a row per request that may be taken")
    reqs = np.empty(cap, dtype=np.int32)
    ends = np.empty(cap, dtype=np.int64)
    pl = np.zeros(cap, dtype=np.int32)
    el = np.zeros(cap, dtype=np.int32)
    qo = np.zeros(cap + 1, dtype=np.int32)
    new = np.empty(max(int(ip[-1]), 1), dtype=np.int32)
    n_new = C.c_int64()
    k = int(check(lib().rt_chunk_prepare(t, n, _ptr(toks), _ptr(ip), _ptr(done), _ptr(held), int(head), int(budget),
                                         _ptr(req_to_token), req_to_token.shape[1], _ptr(pl), _ptr(el), _ptr(qo),
                                         _ptr(new), new.size, _ptr(reqs), _ptr(ends), C.byref(n_new))))
    return reqs[:k], ends[:k], pl[:k], el[:k], qo[:k + 1], new[:n_new.value]


def rt_chunk_finish(t, tok_indptr: np.ndarray, reqs, done: np.ndarray, held: np.ndarray, head: int) -> int:
    """After a launch's kernels: unlock the finished requests' end nodes; the new head."""
    ip = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    rq = _i32(reqs)
    return int(check(lib().rt_chunk_finish(t, int(ip.size - 1), _ptr(ip), _ptr(rq), rq.size, _ptr(done), _ptr(held),
                                           int(head))))


RT_ORDERS = {"fcfs": 0, "lpm": 1}


def rt_serve_round(t, tokens: np.ndarray, tok_indptr: np.ndarray, after, scheduled, window: int, order: str,
                   batch: int) -> np.ndarray:
    """One serve round: the requests picked from the `window` oldest unscheduled ones (ready
    ones only), in arrival order ("fcfs") or longest cached prefix first ("lpm")."""
    if order not in RT_ORDERS:
        raise ValueError(f"unknown scheduling order {order!r}")
    ip = np.ascontiguousarray(tok_indptr, dtype=np.int64)
    n = int(ip.size - 1)
    af = _i32(after)
    sc = np.ascontiguousarray(scheduled, dtype=np.uint8)
    if af.size != n or sc.size != n:
        raise ValueError("rt_serve_round: after and scheduled must hold one entry per request")
    toks = _i32(tokens)
    pick = np.empty(max(int(batch), 1), dtype=np.int32)
    k = int(check(lib().rt_serve_round(t, n, _ptr(toks), _ptr(ip), _ptr(af), _ptr(sc), int(window),
                                       RT_ORDERS[order], int(batch), _ptr(pick))))
    return pick[:k]


# ------------------------------------------------------------------------------------------
# kernels (device); tensors must live on the ROCm device
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    """The HIP stream handle a call is issued on: the given torch stream, else torch's current
    stream on the current device (read as a raw handle; building a Stream object per call
    costs more host time than a small launch)."""
    torch = _torch()
    if stream is not None:
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice()))


def pkv_kv_scatter(k_src, v_src, slots, k_pool, v_pool, k_inv_scale=None, v_inv_scale=None, stream=None) -> None:
    torch = _torch()
    n, hkv, d = k_src.shape
    if v_src.shape != k_src.shape or k_pool.shape != v_pool.shape or tuple(k_pool.shape[1:]) != (hkv, d) \
            or slots.shape != (n,):
        raise ValueError("kv_scatter: shape mismatch")
    args = (_dev(k_src, "k_src", ndim=3), _dev(v_src, "v_src", k_src.dtype, 3), _dtype_code(k_src),
            _dev(slots, "slots", torch.int32, 1), n, _dev(k_pool, "k_pool", ndim=3),
            _dev(v_pool, "v_pool", k_pool.dtype, 3), _dtype_code(k_pool), k_pool.shape[0], hkv, d,
            _dev(k_inv_scale, "k_inv_scale", torch.float32), _dev(v_inv_scale, "v_inv_scale", torch.float32),
            _stream(stream))
    check(lib().pkv_kv_scatter(*args))


def pkv_append_slots(req_to_token, seq_lens, slots, stream=None) -> None:
    torch = _torch()
    b = slots.shape[0]
    if seq_lens.shape != (b,) or req_to_token.dim() != 2 or req_to_token.shape[0] < b:
        raise ValueError("append_slots: shape mismatch")
    check(lib().pkv_append_slots(_dev(req_to_token, "req_to_token", torch.int32), req_to_token.shape[1],
                                 _dev(seq_lens, "seq_lens", torch.int32), _dev(slots, "slots", torch.int32), b,
                                 _stream(stream)))


def pkv_extend_tile(qo_dtype: int, pool_dtype: int, hq: int, hkv: int, d: int) -> int:
    return int(check(lib().pkv_extend_tile(qo_dtype, pool_dtype, hq, hkv, d)))


def pkv_extend_plan(prefix_lens, extend_lens, tile: int) -> np.ndarray:
    pl, el = _i32(prefix_lens), _i32(extend_lens)
    n = int(check(lib().pkv_extend_plan_size(_ptr(el), el.size, int(tile))))
    work = np.empty((max(n, 1), 2), dtype=np.int32)
    check(lib().pkv_extend_plan(_ptr(pl), _ptr(el), el.size, int(tile), _ptr(work), n))
    return work[:n]


def pkv_extend_attention(q, o, k_pool, v_pool, req_to_token, prefix_lens, extend_lens, qo_indptr, work, sm_scale,
                         k_scale=None, v_scale=None, stream=None) -> None:
    torch = _torch()
    tq, hq, d = q.shape
    ns, hkv, d2 = k_pool.shape
    if o.shape != q.shape or o.dtype != q.dtype or v_pool.shape != k_pool.shape or d2 != d:
        raise ValueError("extend: shape mismatch")
    nr = prefix_lens.shape[0]
    if extend_lens.shape != (nr,) or qo_indptr.shape != (nr + 1,) or req_to_token.dim() != 2 \
            or req_to_token.shape[0] < nr or work.dim() != 2 or work.shape[1] != 2:
        raise ValueError("extend: table shape mismatch")
    args = (_dev(q, "q"), _dev(o, "o"), _dtype_code(q), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
            _dtype_code(k_pool), ns, _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
            _dev(req_to_token, "req_to_token", torch.int32), req_to_token.shape[1],
            _dev(prefix_lens, "prefix_lens", torch.int32), _dev(extend_lens, "extend_lens", torch.int32),
            _dev(qo_indptr, "qo_indptr", torch.int32), nr, _dev(work, "work", torch.int32), work.shape[0], hq, hkv, d,
            float(sm_scale), _stream(stream))
    check(lib().pkv_extend_attention(*args))


def pkv_decode_chunk(batch: int, hkv: int, max_seq_len: int) -> int:
    return int(lib().pkv_decode_chunk(batch, hkv, max_seq_len))


def pkv_decode_workspace_bytes(batch: int, hq: int, d: int, max_seq_len: int, chunk: int) -> int:
    return int(lib().pkv_decode_workspace_bytes(batch, hq, d, max_seq_len, chunk))


def pkv_decode_attention(q, o, k_pool, v_pool, req_to_token, seq_lens, max_seq_len, sm_scale, workspace,
                         chunk: int = 0, k_scale=None, v_scale=None, stream=None) -> None:
    torch = _torch()
    b, hq, d = q.shape
    ns, hkv, d2 = k_pool.shape
    if o.shape != q.shape or v_pool.shape != k_pool.shape or d2 != d or seq_lens.shape != (b,) \
            or req_to_token.dim() != 2 or req_to_token.shape[0] < b:
        raise ValueError("decode: shape mismatch")
    args = (_dev(q, "q"), _dev(o, "o", q.dtype), _dtype_code(q), _dev(k_pool, "k_pool"),
            _dev(v_pool, "v_pool", k_pool.dtype), _dtype_code(k_pool), ns, _dev(k_scale, "k_scale", torch.float32),
            _dev(v_scale, "v_scale", torch.float32), _dev(req_to_token, "req_to_token", torch.int32),
            req_to_token.shape[1], _dev(seq_lens, "seq_lens", torch.int32), b, int(max_seq_len), hq, hkv, d,
            float(sm_scale), int(chunk), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream))
    check(lib().pkv_decode_attention(*args))


def pkv_decode_shared_rows(qo_dtype: int, pool_dtype: int, hq: int, hkv: int, d: int) -> int:
    """Member sequences per shared-prefix item for a shape (negative: not supported)."""
    return int(lib().pkv_decode_shared_rows(qo_dtype, pool_dtype, hq, hkv, d))


def pkv_decode_shared_plan(req_to_token: np.ndarray, seq_lens, chunk: int, rows: int, rows_from_tree: bool = False,
                           max_span: int = 1, private_items: bool = False):
    """Host plan of the shared-prefix decode over host slot rows: (members [batch],
    skip [batch], items [n, 4]) as int32 arrays.  rows_from_tree: the rows come from one
    radix tree, so each chunk's last slot decides it (otherwise every slot is compared);
    max_span: chunks one item may span; private_items: one-member items also cover every
    sequence's remaining chunks (skip then reaches each context's end)."""
    r2t = _i32(req_to_token)
    sl = _i32(seq_lens)
    b = int(sl.size)
    if r2t.ndim != 2 or r2t.shape[0] < b:
        raise ValueError("decode plan: req_to_token must be [>= batch, stride]")
    members = np.empty(max(b, 1), dtype=np.int32)
    skip = np.empty(max(b, 1), dtype=np.int32)
    # a job holds two members or more, so it makes at most members / 2 items when an item
    # takes two or more rows (members per item); with one row per item, one item per member
    cap = max(b * (r2t.shape[1] // max(int(chunk), 1)) // (2 if rows >= 2 else 1) + 1, 1)
    if private_items and chunk > 0:     # at most one private item per chunk of each context
        cap += int(((sl.astype(np.int64) + chunk - 1) // chunk).sum())
    items = np.empty((cap, 4), dtype=np.int32)
    n = int(check(lib().pkv_decode_shared_plan(_ptr(r2t), r2t.shape[1], _ptr(sl), b, int(chunk), int(rows),
                                               int(max_span), int(bool(rows_from_tree)), int(bool(private_items)),
                                               _ptr(members), _ptr(skip), _ptr(items), cap)))
    return members[:b], skip[:b], items[:n]


def pkv_decode_first_split(skip, seq_lens, chunk: int) -> int:
    """First chunk the split phase must launch for a plan's skip at the current lengths, or
    PKV_NO_SPLIT_PHASE."""
    sk, sl = _i32(skip), _i32(seq_lens)
    if sk.size != sl.size:
        raise ValueError("first split: skip and seq_lens differ in length")
    return int(check(lib().pkv_decode_first_split(_ptr(sk), _ptr(sl), sl.size, int(chunk))))


def pkv_decode_plan(req_to_token: np.ndarray, seq_lens, chunk: int, rows: int, hkv: int,
                    resident_workgroups: int, private_max_workgroups: int):
    """The shared-prefix plan with the library's choices (spans, private items) over host slot
    rows from one radix tree: (members, skip, items [n, 4], first_split), or None when nothing
    is shared."""
    r2t = _i32(req_to_token)
    sl = _i32(seq_lens)
    b = int(sl.size)
    if r2t.ndim != 2 or r2t.shape[0] < b:
        raise ValueError("decode plan: req_to_token must be [>= batch, stride]")
    cap = int(check(lib().pkv_decode_plan_items_cap(_ptr(sl), b, r2t.shape[1], int(chunk), int(rows))))
    members = np.empty(max(b, 1), dtype=np.int32)
    skip = np.empty(max(b, 1), dtype=np.int32)
    items = np.empty((max(cap, 1), 4), dtype=np.int32)
    first = C.c_int32()
    n = int(check(lib().pkv_decode_plan(_ptr(r2t), r2t.shape[1], _ptr(sl), b, int(chunk), int(rows), int(hkv),
                                        int(resident_workgroups), int(private_max_workgroups), _ptr(members),
                                        _ptr(skip), _ptr(items), cap, C.byref(first))))
    if n == 0:
        return None
    return members[:b], skip[:b], items[:n], int(first.value)


def pkv_decode_attention_shared(q, o, k_pool, v_pool, req_to_token, seq_lens, max_seq_len, sm_scale, workspace,
                                chunk: int, members, skip, items, first_split: int = 0, k_scale=None, v_scale=None,
                                stream=None) -> None:
    """pkv_decode_attention with a shared-prefix plan (device int32 members [b], skip [b],
    items [n, 4] from pkv_decode_shared_plan for the same rows and chunk; first_split = the
    smallest skip, or 0)."""
    torch = _torch()
    b, hq, d = q.shape
    ns, hkv, d2 = k_pool.shape
    if o.shape != q.shape or v_pool.shape != k_pool.shape or d2 != d or seq_lens.shape != (b,) \
            or req_to_token.dim() != 2 or req_to_token.shape[0] < b:
        raise ValueError("decode: shape mismatch")
    if members.shape != (b,) or skip.shape != (b,) or items.dim() != 2 or items.shape[1] != 4:
        raise ValueError("decode: plan shape mismatch")
    args = (_dev(q, "q"), _dev(o, "o", q.dtype), _dtype_code(q), _dev(k_pool, "k_pool"),
            _dev(v_pool, "v_pool", k_pool.dtype), _dtype_code(k_pool), ns, _dev(k_scale, "k_scale", torch.float32),
            _dev(v_scale, "v_scale", torch.float32), _dev(req_to_token, "req_to_token", torch.int32),
            req_to_token.shape[1], _dev(seq_lens, "seq_lens", torch.int32), b, int(max_seq_len), hq, hkv, d,
            float(sm_scale), int(chunk), _dev(members, "members", torch.int32), _dev(skip, "skip", torch.int32),
            _dev(items, "items", torch.int32), items.shape[0], int(first_split), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    check(lib().pkv_decode_attention_shared(*args))


def pkv_decode_attention_static(q, o, k_pool, v_pool, req_to_token, seq_lens, max_seq_len, sm_scale,
                                chunk: int = 0, members=None, skip=None, items=None, first_split: int = 0,
                                k_scale=None, v_scale=None, stream=None) -> None:
    """pkv_decode_attention (or, with a plan, pkv_decode_attention_shared) with the partials in
    the library's static device array instead of a workspace: allocates nothing."""
    torch = _torch()
    b, hq, d = q.shape
    ns, hkv, d2 = k_pool.shape
    if o.shape != q.shape or v_pool.shape != k_pool.shape or d2 != d or seq_lens.shape != (b,) \
            or req_to_token.dim() != 2 or req_to_token.shape[0] < b:
        raise ValueError("decode: shape mismatch")
    if items is None:
        if members is not None or skip is not None:
            raise ValueError("decode: members and skip come with items")
        n_items = 0
    else:
        if members is None or skip is None or members.shape != (b,) or skip.shape != (b,) or items.dim() != 2 \
                or items.shape[1] != 4:
            raise ValueError("decode: plan shape mismatch")
        n_items = items.shape[0]
    args = (_dev(q, "q"), _dev(o, "o", q.dtype), _dtype_code(q), _dev(k_pool, "k_pool"),
            _dev(v_pool, "v_pool", k_pool.dtype), _dtype_code(k_pool), ns, _dev(k_scale, "k_scale", torch.float32),
            _dev(v_scale, "v_scale", torch.float32), _dev(req_to_token, "req_to_token", torch.int32),
            req_to_token.shape[1], _dev(seq_lens, "seq_lens", torch.int32), b, int(max_seq_len), hq, hkv, d,
            float(sm_scale), int(chunk), _dev(members, "members", torch.int32), _dev(skip, "skip", torch.int32),
            _dev(items, "items", torch.int32), n_items, int(first_split), _stream(stream))
    check(lib().pkv_decode_attention_static(*args))
