"""Oracle attention in float64, recomputed from each request's full token sequence.  TEST INFRASTRUCTURE ONLY.

The pages state only that the matched prefix's K/V is reused and that the rest of
the prompt is prefilled (RadixAttention explainer, "プレフィックスマッチングアルゴリズム";
overview page, "Why this matters in production").  The attention itself is the
textbook scaled dot product, which is what a reused prefix must reproduce exactly:
for query position i of a request and query head h, with kv head g = h // (Hq/Hkv),

    s_j = scale * <q_i,h , k_j,g>        for j <= i (full over the prefix, causal over the suffix)
    p   = exp(s - max s) / sum exp(s - max s)
    o_i,h = sum_j p_j v_j,g

K/V rows come straight from the value table by token position, with no tree and
no slots ("no reuse"), in the precision they are stored in: float32, bf16, or the
fp8 code times its per-head scale.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import fp8


def stored_kv(values_f32: np.ndarray, pool_dtype: str, inv_scale=None, scale=None) -> np.ndarray:
    """float64 K or V rows [n, hkv, d] as the pool holds them."""
    if pool_dtype in ("f32", "bf16"):
        # the source rows are already in their stored precision (bf16 values are exact in float32)
        return np.asarray(values_f32, dtype=np.float64)
    if pool_dtype == "fp8_e4m3":
        inv = np.asarray(inv_scale, dtype=np.float32)[None, :, None]
        codes = fp8.quantise(values_f32, inv)
        return fp8.dequantise(codes, np.asarray(scale, dtype=np.float64)[None, :, None])
    raise ValueError(pool_dtype)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions: Sequence[int], scale: float) -> np.ndarray:
    """Attention of query rows ``q`` [n, hq, d] at token positions ``positions`` over k, v [L, hkv, d].

    Query row r attends keys 0..positions[r].  Returns float64 [n, hq, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    group = hq // hkv
    pos = np.asarray(positions, dtype=np.int64)
    visible = np.arange(L)[None, :] <= pos[:, None]          # [n, L]
    out = np.empty((n, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        s = scale * (q[:, h, :] @ k[:, g, :].T)               # [n, L]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def request_kv(wl, rows: np.ndarray):
    """float64 K and V [L, hkv, d] for canonical value rows, as stored in the workload's pool."""
    vt = wl.values
    k = stored_kv(vt.k(rows), wl.shape.pool_dtype, wl.k_inv_scale, wl.k_scale)
    v = stored_kv(vt.v(rows), wl.shape.pool_dtype, wl.v_inv_scale, wl.v_scale)
    return k, v


def extend_rows(wl, req, prefix_len: int, sample: Optional[Sequence[int]] = None) -> np.ndarray:
    """Oracle output for the extend positions [prefix_len, L) of one request (or a sample of them)."""
    L = len(req.tokens)
    pos = np.arange(prefix_len, L) if sample is None else np.asarray(sample, dtype=np.int64)
    hi = int(pos.max()) + 1 if pos.size else 0
    k, v = request_kv(wl, req.rows[:hi])
    q = wl.values.q(req.rows[pos])
    return attend(q, k, v, pos, wl.shape.sm_scale)


def decode_row(wl, rows: np.ndarray) -> np.ndarray:
    """Oracle output [hq, d] for the newest token of a sequence whose value rows are ``rows``."""
    k, v = request_kv(wl, rows)
    q = wl.values.q(rows[-1:])
    return attend(q, k, v, [len(rows) - 1], wl.shape.sm_scale)[0]
