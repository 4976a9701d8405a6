"""Pins for the float64 oracle attention: closed forms, PyTorch's float64 scaled-dot-product
attention (a library routine) with repeated KV heads, prefix/suffix offsets, and decode."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oa


def sdpa_rows(q, k, v, positions, scale):
    """torch float64 attention on the CPU: query row r sees keys 0..positions[r]."""
    q = torch.from_numpy(np.asarray(q, dtype=np.float64)).permute(1, 0, 2)      # [hq, n, d]
    k = torch.from_numpy(np.asarray(k, dtype=np.float64)).permute(1, 0, 2)      # [hkv, L, d]
    v = torch.from_numpy(np.asarray(v, dtype=np.float64)).permute(1, 0, 2)
    group = q.shape[0] // k.shape[0]
    k = k.repeat_interleave(group, dim=0)
    v = v.repeat_interleave(group, dim=0)
    L = k.shape[1]
    mask = torch.arange(L)[None, :] <= torch.as_tensor(positions)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,d,L,p", [(8, 8, 64, 80, 0), (8, 8, 64, 80, 64), (32, 8, 128, 300, 250),
                                          (64, 8, 128, 97, 33), (4, 1, 16, 5, 4)])
def test_matches_torch_sdpa(hq, hkv, d, L, p):
    rng = np.random.default_rng(hq * 1000 + L)
    q = rng.standard_normal((L - p, hq, d))
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    pos = np.arange(p, L)
    got = oa.attend(q, k, v, pos, 1 / math.sqrt(d))
    ref = sdpa_rows(q, k, v, pos, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_sharp_softmax_matches_torch():
    # large logits: a missing max subtraction overflows exp
    rng = np.random.default_rng(5)
    q = 40 * rng.standard_normal((20, 4, 32))
    k = rng.standard_normal((50, 2, 32))
    v = rng.standard_normal((50, 2, 32))
    pos = np.arange(30, 50)
    got = oa.attend(q, k, v, pos, 1.0)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, sdpa_rows(q, k, v, pos, 1.0), rtol=0, atol=1e-10)


def test_context_of_one_returns_v():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    o = oa.attend(q, k, v, [0], 0.3)
    np.testing.assert_array_equal(o[0], np.repeat(v[0], 2, axis=0))


def test_equal_keys_average_visible_values():
    rng = np.random.default_rng(2)
    L = 12
    k = np.repeat(rng.standard_normal((1, 2, 8)), L, axis=0)
    v = rng.standard_normal((L, 2, 8))
    q = rng.standard_normal((L, 2, 8))
    o = oa.attend(q, k, v, np.arange(L), 0.5)
    for i in range(L):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), rtol=0, atol=1e-13)


def test_zero_query_is_running_mean():
    rng = np.random.default_rng(3)
    L = 9
    k = rng.standard_normal((L, 1, 4))
    v = rng.standard_normal((L, 1, 4))
    o = oa.attend(np.zeros((L, 3, 4)), k, v, np.arange(L), 1.0)
    for i in range(L):
        for h in range(3):
            np.testing.assert_allclose(o[i, h], v[: i + 1, 0].mean(axis=0), rtol=0, atol=1e-13)


def test_gqa_head_grouping_is_contiguous():
    # kv head g serves query heads g*group .. g*group+group-1; zero a kv head's V and check which q heads see zeros
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 8, 16))
    k = rng.standard_normal((3, 2, 16))
    v = rng.standard_normal((3, 2, 16))
    v[:, 1] = 0
    o = oa.attend(q, k, v, [0, 1, 2], 0.25)
    assert np.all(o[:, 4:] == 0) and np.all(np.abs(o[:, :4]).sum(axis=-1) > 0)


def test_reuse_equals_no_reuse_on_workload():
    # rows [p, L) computed as an extend over a cached prefix equal the same rows of a full prefill
    import workloads
    wl = workloads.tiny_f32()
    req = wl.batches[0][1]
    L = len(req.tokens)
    ext = oa.extend_rows(wl, req, 64)
    full = oa.extend_rows(wl, req, 0)
    np.testing.assert_allclose(ext, full[64:], rtol=0, atol=1e-12)
    k, v = oa.request_kv(wl, req.rows)
    ref = sdpa_rows(wl.values.q(req.rows), k, v, np.arange(L), wl.shape.sm_scale)
    np.testing.assert_allclose(full, ref, rtol=0, atol=1e-12)


def test_decode_row_is_last_causal_row():
    import workloads
    wl = workloads.tiny_f32()
    req = wl.batches[0][0]
    full = oa.extend_rows(wl, req, 0)
    np.testing.assert_allclose(oa.decode_row(wl, req.rows), full[-1], rtol=0, atol=1e-12)


def test_stored_fp8_kv_matches_torch_float8():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 4, 32)).astype(np.float32)
    scale = (np.abs(x).max(axis=(0, 2)) / np.float32(448)).astype(np.float32)
    inv = (np.float32(1) / scale).astype(np.float32)
    got = oa.stored_kv(x, "fp8_e4m3", inv, scale)
    prod = torch.from_numpy(x) * torch.from_numpy(inv)[None, :, None]
    ref = prod.to(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(scale).double()[None, :, None]
    np.testing.assert_array_equal(got, ref.numpy())
