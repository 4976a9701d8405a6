"""Argument validation of the kernel entry points, on the CPU: every rejected call returns its
documented error code before any HIP call is made (fake, never dereferenced device pointers),
and empty calls return 0 without launching anything."""
import ctypes as C

import pytest

import prefix_shared_kv_match_amd as pkv
from prefix_shared_kv_match_amd import PKV_BF16, PKV_F32, PKV_FP8_E4M3

INVAL, UNSUP = -1, -7
P = C.c_void_p(0x10000)          # stands in for a device pointer; no test below reaches a launch


def extend(**kw):
    a = dict(q=P, o=P, qo=PKV_BF16, kp=P, vp=P, pool=PKV_BF16, num_slots=1024, ks=None, vs=None, r2t=P, stride=64,
             pl=P, el=P, qo_indptr=P, num_reqs=4, work=P, n_work=8, hq=32, hkv=8, d=128, sm=0.088, stream=None)
    a.update(kw)
    return pkv.lib().pkv_extend_attention(a["q"], a["o"], a["qo"], a["kp"], a["vp"], a["pool"], a["num_slots"], a["ks"],
                                          a["vs"], a["r2t"], a["stride"], a["pl"], a["el"], a["qo_indptr"],
                                          a["num_reqs"], a["work"], a["n_work"], a["hq"], a["hkv"], a["d"], a["sm"],
                                          a["stream"])


def decode(**kw):
    a = dict(q=P, o=P, qo=PKV_BF16, kp=P, vp=P, pool=PKV_BF16, num_slots=1024, ks=None, vs=None, r2t=P, stride=4096,
             lens=P, batch=4, max_len=4096, hq=32, hkv=8, d=128, sm=0.088, chunk=256, ws=P, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return pkv.lib().pkv_decode_attention(a["q"], a["o"], a["qo"], a["kp"], a["vp"], a["pool"], a["num_slots"],
                                          a["ks"], a["vs"], a["r2t"], a["stride"], a["lens"], a["batch"],
                                          a["max_len"], a["hq"], a["hkv"], a["d"], a["sm"], a["chunk"], a["ws"],
                                          a["ws_bytes"], a["stream"])


def decode_shared(**kw):
    a = dict(q=P, o=P, qo=PKV_BF16, kp=P, vp=P, pool=PKV_BF16, num_slots=1024, ks=None, vs=None, r2t=P, stride=4096,
             lens=P, batch=4, max_len=4096, hq=32, hkv=8, d=128, sm=0.088, chunk=256, members=P, skip=P, items=P,
             n_items=3, first_split=0, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return pkv.lib().pkv_decode_attention_shared(
        a["q"], a["o"], a["qo"], a["kp"], a["vp"], a["pool"], a["num_slots"], a["ks"], a["vs"], a["r2t"], a["stride"],
        a["lens"], a["batch"], a["max_len"], a["hq"], a["hkv"], a["d"], a["sm"], a["chunk"], a["members"], a["skip"],
        a["items"], a["n_items"], a["first_split"], a["ws"], a["ws_bytes"], a["stream"])


def scatter(**kw):
    a = dict(ks=P, vs=P, src=PKV_BF16, slots=P, n=16, kp=P, vp=P, pool=PKV_BF16, num_slots=1024, hkv=8, d=128,
             kinv=None, vinv=None, stream=None)
    a.update(kw)
    return pkv.lib().pkv_kv_scatter(a["ks"], a["vs"], a["src"], a["slots"], a["n"], a["kp"], a["vp"], a["pool"],
                                    a["num_slots"], a["hkv"], a["d"], a["kinv"], a["vinv"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=30), INVAL),                       # hq not a multiple of hkv
    (dict(num_reqs=-1), INVAL),
    (dict(stride=0), INVAL),
    (dict(q=None), INVAL),
    (dict(d=96), UNSUP),                        # head dims 64 and 128 only
    (dict(hq=24, hkv=8), UNSUP),                # group size 3
    (dict(pool=PKV_FP8_E4M3), INVAL),           # fp8 pool without scales
    (dict(sm=0.0), INVAL),
    (dict(hq=64, hkv=64), UNSUP),               # a 64-head bf16 slot (16 KiB) is wider than a buffer record
    (dict(num_reqs=40000, stride=16384), UNSUP),  # slot table beyond 32-bit buffer offsets
])
def test_extend_rejects(kw, code):
    assert extend(**kw) == code
    assert pkv.lib().pkv_last_error()


def test_extend_empty_is_a_no_op():
    assert extend(n_work=0) == 0
    assert extend(n_work=0, q=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(hq=30), INVAL),
    (dict(max_len=8192), INVAL),                # longer than the table stride
    (dict(chunk=100), INVAL),                   # not a multiple of 64
    (dict(ws_bytes=16), INVAL),                 # workspace too small
    (dict(pool=PKV_FP8_E4M3), INVAL),           # fp8 pool without scales
    (dict(ws=None), INVAL),
    (dict(d=96), UNSUP),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def test_decode_empty_batch_is_a_no_op():
    assert decode(batch=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(members=None), INVAL),                # a plan without its arrays
    (dict(items=None), INVAL),
    (dict(chunk=0), INVAL),                     # a plan is made for one chunk size
    (dict(n_items=-1), INVAL),
    (dict(qo=PKV_F32, pool=PKV_F32), UNSUP),    # no shared-prefix kernel for fp32
    (dict(hq=24, hkv=8), UNSUP),                # group size 3: no shared-prefix kernel
    (dict(max_len=8192), INVAL),                # longer than the table stride, as without a plan
])
def test_decode_shared_rejects(kw, code):
    assert decode_shared(**kw) == code
    assert pkv.lib().pkv_last_error()


def test_decode_shared_without_items_is_plain_decode_validation():
    # no items: the same checks as pkv_decode_attention (and no launch for an empty batch)
    assert decode_shared(n_items=0, members=None, skip=None, items=None, batch=0) == 0
    assert decode_shared(n_items=0, members=None, skip=None, items=None, ws=None) == INVAL


def test_decode_shared_rows():
    lib = pkv.lib()
    assert lib.pkv_decode_shared_rows(PKV_BF16, PKV_BF16, 32, 8, 128) == 32
    assert lib.pkv_decode_shared_rows(PKV_BF16, PKV_FP8_E4M3, 64, 8, 128) == 16
    assert lib.pkv_decode_shared_rows(PKV_BF16, PKV_BF16, 32, 32, 128) == 128
    assert lib.pkv_decode_shared_rows(PKV_F32, PKV_F32, 8, 8, 64) == UNSUP
    assert lib.pkv_decode_shared_rows(PKV_BF16, PKV_BF16, 30, 8, 128) == INVAL


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), INVAL),
    (dict(hkv=0), INVAL),
    (dict(slots=None), INVAL),
    (dict(d=96), UNSUP),
    (dict(src=PKV_F32, pool=PKV_BF16), UNSUP),
    (dict(pool=PKV_FP8_E4M3), INVAL),           # fp8 pool without inverse scales
])
def test_scatter_rejects(kw, code):
    assert scatter(**kw) == code


def test_scatter_and_append_empty_are_no_ops():
    assert scatter(n=0) == 0
    assert pkv.lib().pkv_append_slots(P, 64, P, P, 0, None) == 0
    assert pkv.lib().pkv_append_slots(P, 64, P, P, -1, None) == INVAL


def test_workspace_and_chunk_helpers():
    lib = pkv.lib()
    assert lib.pkv_decode_workspace_bytes(0, 32, 128, 4096, 256) == 0
    need = lib.pkv_decode_workspace_bytes(4, 32, 128, 4096, 256)
    assert need == 4 * 32 * 16 * (2 + 128) * 4
    for b in (1, 64, 512):
        c = lib.pkv_decode_chunk(b, 8, 8192)
        assert 128 <= c <= 1024 and c % 64 == 0
    # the all-heads kernel (hkv 2, 4, 8) launches one workgroup per (sequence, chunk): halve the
    # chunk until 2048 of them are launched (64 x 2,000-token few-shot sequences: 128-token
    # chunks; 16 x 33,856: 256; 512 x 8,224: 1,024); per-head kernels count kv heads too
    assert lib.pkv_decode_chunk(64, 8, 2000) == 128
    assert lib.pkv_decode_chunk(16, 8, 33856) == 256
    assert lib.pkv_decode_chunk(512, 8, 8224) == 1024
    assert lib.pkv_decode_chunk(256, 32, 1897) == 1024
    assert lib.pkv_decode_chunk(4, 32, 1000) == 128
    assert lib.pkv_extend_tile(PKV_BF16, PKV_BF16, 32, 8, 128) == 32
    assert lib.pkv_extend_tile(PKV_BF16, PKV_BF16, 32, 32, 128) == 128
    assert lib.pkv_extend_tile(PKV_F32, PKV_F32, 8, 8, 64) > 0
    assert lib.pkv_extend_tile(PKV_BF16, PKV_BF16, 24, 8, 128) == UNSUP
    # head dim 64 with bf16 q/o: the VALU kernel, 16 query tokens per work item, any group size
    assert lib.pkv_extend_tile(PKV_BF16, PKV_BF16, 32, 8, 64) == 16
    assert lib.pkv_extend_tile(PKV_BF16, PKV_FP8_E4M3, 24, 8, 64) == 16
    assert lib.pkv_extend_tile(PKV_BF16, PKV_BF16, 32, 8, 96) == UNSUP
