"""Decode with no allocation: pkv_decode_attention_static (partials in the library's static
device array) against pkv_decode_attention / pkv_decode_attention_shared (caller workspace).

Both run the same kernels at the same chunk and plan, so their outputs must be bit-identical.
Two calls in a row, the second smaller, show that the array's leftover partials from one call
never reach the next; a plain decode with the automatic chunk, one whose automatic chunk the
static call has to double, and one whose partials cannot fit (an error before any launch) cover
the size handling."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_shared_kv_match_amd as pkv
    pkv.lib()


def log(msg):
    print(msg, flush=True)


def make_rows(rng, seq_lens, group, prefix_len, stride, perm):
    """Slot rows as one radix tree would hand them out: requests in groups of `group` share
    their first `prefix_len` slots; every other position has a slot of its own."""
    b = len(seq_lens)
    r2t = np.zeros((b, stride), dtype=np.int32)
    nxt = 0
    for g0 in range(0, b, group):
        pre = perm[nxt:nxt + prefix_len]
        nxt += prefix_len
        for i in range(g0, min(g0 + group, b)):
            r2t[i, :prefix_len] = pre
            own = int(seq_lens[i]) - prefix_len
            r2t[i, prefix_len:seq_lens[i]] = perm[nxt:nxt + own]
            nxt += own
    assert nxt <= len(perm)
    return r2t


class Pools:
    def __init__(self, pool, num_slots, seed):
        g = torch.Generator(device="cpu").manual_seed(seed)
        self.pool = pool
        self.num_slots = num_slots
        if pool == "bf16":
            self.k = (torch.randn(num_slots, HKV, D, generator=g) * 0.5).bfloat16().cuda()
            self.v = torch.randn(num_slots, HKV, D, generator=g).bfloat16().cuda()
            self.ks = self.vs = None
        else:
            # random E4M3 codes with the two NaN codes (0x7F, 0xFF) replaced by zero
            codes = torch.randint(0, 256, (2, num_slots, HKV, D), generator=g, dtype=torch.uint8)
            codes[(codes & 0x7F) == 0x7F] = 0
            self.k, self.v = codes[0].cuda(), codes[1].cuda()
            self.ks = (torch.rand(HKV, generator=g) * 0.02 + 0.01).cuda()
            self.vs = (torch.rand(HKV, generator=g) * 0.02 + 0.01).cuda()


def case_inputs(rng, batch, ctx, group, prefix_len, stride, num_slots):
    seq_lens = rng.integers(ctx[0], ctx[1] + 1, size=batch).astype(np.int32)
    seq_lens = np.maximum(seq_lens, prefix_len + 1)
    perm = rng.permutation(num_slots).astype(np.int32)
    r2t = make_rows(rng, seq_lens, group, prefix_len, stride, perm)
    q = torch.from_numpy(rng.standard_normal((batch, HQ, D)).astype(np.float32)).bfloat16().cuda()
    return seq_lens, r2t, q


def run_pair(pkv, pools, seq_lens, r2t, q, chunk, max_len=None, plan=False):
    """One static call and one workspace call on the same inputs; returns both outputs."""
    b = len(seq_lens)
    max_len = int(seq_lens.max()) if max_len is None else max_len
    sm = 1.0 / math.sqrt(D)
    r2t_d = torch.from_numpy(r2t).cuda()
    sl_d = torch.from_numpy(seq_lens).cuda()
    o_static = torch.full_like(q, float("nan"))
    o_ws = torch.full_like(q, float("nan"))
    ws_chunk = chunk if chunk else pkv.pkv_decode_chunk(b, HKV, max_len)
    args = (pools.k, pools.v, r2t_d, sl_d, max_len, sm)
    if plan:
        rows = pkv.pkv_decode_shared_rows(pkv.PKV_BF16, pkv.PKV_BF16 if pools.pool == "bf16" else pkv.PKV_FP8_E4M3,
                                          HQ, HKV, D)
        assert rows > 0
        p = pkv.pkv_decode_plan(r2t, seq_lens, ws_chunk, rows, HKV, 16, 1 << 20)
        assert p is not None, "no shared items"
        members, skip, items, first = p
        dm = torch.from_numpy(np.ascontiguousarray(members)).cuda()
        ds = torch.from_numpy(np.ascontiguousarray(skip)).cuda()
        di = torch.from_numpy(np.ascontiguousarray(items)).cuda()
        pkv.pkv_decode_attention_static(q, o_static, *args, chunk=ws_chunk, members=dm, skip=ds, items=di,
                                        first_split=first, k_scale=pools.ks, v_scale=pools.vs)
        ws = torch.empty(pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, ws_chunk), dtype=torch.uint8,
                         device="cuda")
        pkv.pkv_decode_attention_shared(q, o_ws, *args, ws, ws_chunk, dm, ds, di, first_split=first,
                                        k_scale=pools.ks, v_scale=pools.vs)
    else:
        pkv.pkv_decode_attention_static(q, o_static, *args, chunk=chunk, k_scale=pools.ks, v_scale=pools.vs)
        ws = torch.empty(pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, ws_chunk), dtype=torch.uint8,
                         device="cuda")
        pkv.pkv_decode_attention(q, o_ws, *args, ws, ws_chunk, k_scale=pools.ks, v_scale=pools.vs)
    torch.cuda.synchronize()
    return o_static, o_ws


def assert_same(o_static, o_ws, what):
    assert not torch.isnan(o_ws).any(), f"{what}: workspace decode left rows unwritten"
    diff = (o_static.float() - o_ws.float()).abs().max().item()
    log(f"{what}: max |static - workspace| = {diff}")
    assert torch.equal(o_static, o_ws), f"{what}: outputs differ (max |d| {diff})"


@pytest.mark.parametrize("pool", ["bf16", "fp8"])
@pytest.mark.parametrize("plan", [False, True])
def test_static_decode_matches_workspace_decode_twice(pool, plan):
    import prefix_shared_kv_match_amd as pkv
    log(f"static decode: pool {pool}, plan {plan}")
    rng = np.random.default_rng(1234 + (pool == "fp8") + 2 * plan)
    pools = Pools(pool, 200_000, seed=7)
    # first call: 48 sequences of 600..3000 tokens, groups of 8 sharing 1,024 tokens
    sl, r2t, q = case_inputs(rng, 48, (600, 3000), 8, 1024, 3072, pools.num_slots)
    assert_same(*run_pair(pkv, pools, sl, r2t, q, 128, plan=plan), f"{pool} plan={plan} call 1 (48 seqs)")
    # second call, smaller: 6 sequences of 200..900 tokens sharing 128 tokens in pairs
    sl, r2t, q = case_inputs(rng, 6, (200, 900), 2, 128, 1024, pools.num_slots)
    assert_same(*run_pair(pkv, pools, sl, r2t, q, 128, plan=plan), f"{pool} plan={plan} call 2 (6 seqs)")


def test_static_decode_automatic_chunk_and_doubling():
    import prefix_shared_kv_match_amd as pkv
    log("static decode: automatic chunk")
    rng = np.random.default_rng(99)
    pools = Pools("bf16", 120_000, seed=8)
    # the automatic chunk fits the array as it is
    sl, r2t, q = case_inputs(rng, 40, (300, 2500), 4, 256, 2560, pools.num_slots)
    b, max_len = len(sl), int(sl.max())
    assert pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, pkv.pkv_decode_chunk(b, HKV, max_len)) \
        <= pkv.PKV_DECODE_STATIC_SCRATCH_BYTES
    assert_same(*run_pair(pkv, pools, sl, r2t, q, 0), "automatic chunk")
    # 64 sequences under a 65,536-token bound: the automatic chunk (1,024) needs more than the
    # array holds, so the static call doubles it; the workspace call is given the doubled chunk
    sl, r2t, q = case_inputs(rng, 64, (100, 1500), 4, 64, 65536, pools.num_slots)
    b, max_len = 64, 65536
    auto = pkv.pkv_decode_chunk(b, HKV, max_len)
    assert pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, auto) > pkv.PKV_DECODE_STATIC_SCRATCH_BYTES
    chunk = auto
    while pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, chunk) > pkv.PKV_DECODE_STATIC_SCRATCH_BYTES:
        chunk *= 2
    o_static = torch.full_like(q, float("nan"))
    r2t_d, sl_d = torch.from_numpy(r2t).cuda(), torch.from_numpy(sl).cuda()
    sm = 1.0 / math.sqrt(D)
    pkv.pkv_decode_attention_static(q, o_static, pools.k, pools.v, r2t_d, sl_d, max_len, sm)
    o_ws = torch.full_like(q, float("nan"))
    ws = torch.empty(pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, chunk), dtype=torch.uint8, device="cuda")
    pkv.pkv_decode_attention(q, o_ws, pools.k, pools.v, r2t_d, sl_d, max_len, sm, ws, chunk)
    torch.cuda.synchronize()
    assert_same(o_static, o_ws, f"doubled chunk {chunk}")


def test_static_decode_rejects_partials_beyond_the_array():
    import prefix_shared_kv_match_amd as pkv
    b, max_len, chunk = 256, 65536, 64
    assert pkv.pkv_decode_workspace_bytes(b, HQ, D, max_len, chunk) > pkv.PKV_DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros(b, HQ, D, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    kp = torch.zeros(16, HKV, D, dtype=torch.bfloat16, device="cuda")
    r2t = torch.zeros(b, max_len, dtype=torch.int32, device="cuda")
    sl = torch.ones(b, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError, match="static scratch array"):
        pkv.pkv_decode_attention_static(q, o, kp, kp, r2t, sl, max_len, 0.1, chunk=chunk)
    torch.cuda.synchronize()
