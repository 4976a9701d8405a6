"""GPU parity: the HIP path through the C ABI against the oracle, element by element.

Small cases compare every output row; the full-size workloads (in the launch configuration the
bench uses) compare seeded samples of rows that always include each request's first and last
extend row.  Tolerances: fp32 max|d| <= 1e-4; bf16 max|d| <= 2e-2 and relative RMS <= 5e-3;
kv_scatter and every host table bit-exact."""
import math

import numpy as np
import pytest

import workloads
from oracle import attention as oa
from oracle import fp8 as ofp8

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_harness import Run, compare, log, make_engine, src_tensor  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_shared_kv_match_amd as pkv
    pkv.lib()


def report(name, stats):
    worst = max(stats, key=lambda s: s["rel_rms"]) if stats else {}
    log(f"{name}: {len(stats)} checks, worst {worst}")


# ---------------------------------------------------------------------------------------------
# kv_scatter
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("pool", ["f32", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("d", [64, 128])
def test_kv_scatter_bit_exact(pool, d):
    import prefix_shared_kv_match_amd as pkv
    log(f"kv_scatter pool={pool} d={d}")
    rng = np.random.default_rng(d)
    n, hkv, slots_total = 777, 8, 4096
    src = rng.standard_normal((n, hkv, d)).astype(np.float32)
    src_v = rng.standard_normal((n, hkv, d)).astype(np.float32) * 3
    src_v[0, 0, :4] = [0.0, -0.0, -1e-9, 1e6]          # zero, negative zero, tiny negative, saturating
    if pool != "f32":
        src = workloads.round_to_bf16(src)
        src_v = workloads.round_to_bf16(src_v)
    slots = rng.permutation(slots_total)[:n].astype(np.int32)
    sdt = torch.float32 if pool == "f32" else torch.bfloat16
    pdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}[pool]
    kp = torch.zeros((slots_total, hkv, d), dtype=pdt, device="cuda")
    vp = torch.zeros_like(kp)
    ks = vs = kinv = vinv = None
    if pool == "fp8_e4m3":
        ks = (np.abs(src).max(axis=(0, 2)) / 448).astype(np.float32)
        vs = (np.abs(src_v[1:]).max(axis=(0, 2)) / 448).astype(np.float32)
        kinv, vinv = (np.float32(1) / ks).astype(np.float32), (np.float32(1) / vs).astype(np.float32)
    t = lambda a: None if a is None else torch.from_numpy(a).cuda()
    pkv.pkv_kv_scatter(torch.from_numpy(src).to(sdt).cuda(), torch.from_numpy(src_v).to(sdt).cuda(),
                       t(slots), kp, vp, t(kinv), t(vinv))
    torch.cuda.synchronize()
    for pool_t, x, inv in ((kp, src, kinv), (vp, src_v, vinv)):
        got = pool_t.cpu()[torch.from_numpy(slots.astype(np.int64))]
        if pool == "fp8_e4m3":
            np.testing.assert_array_equal(got.numpy(), ofp8.quantise(x, inv[None, :, None]))
        else:
            np.testing.assert_array_equal(got.float().numpy(), x)
    # untouched slots stay zero
    mask = np.ones(slots_total, dtype=bool)
    mask[slots] = False
    assert torch.count_nonzero(kp.cpu()[torch.from_numpy(mask)]).item() == 0


# ---------------------------------------------------------------------------------------------
# small workloads: every row
# ---------------------------------------------------------------------------------------------

def test_tiny_f32_every_row():
    log("tiny_f32")
    r = Run(workloads.tiny_f32(), check_pool=True)
    stats = r.run()
    report("tiny_f32", stats)
    assert stats and stats[0]["max_abs"] <= 1e-4


def test_fewshot_small_every_row():
    log("fewshot small")
    wl = workloads.fewshot_bf16(n_req=8, prefix_len=300, suffix_range=(20, 90), decode_steps=3)
    stats = Run(wl, check_pool=True).run()
    report("fewshot small", stats)


def test_multiturn_small_every_row_with_eviction():
    log("multiturn small")
    # 8 requests of at most 768 tokens stay pinned at once, so 8,000 slots never deadlock, while the
    # conversations hold more unique tokens than that, so LRU eviction fires
    wl = workloads.multiturn_bf16(n_conv=24, turns=4, turn_range=(16, 96), batch=8, pool_slots=20000,
                                  capacity=8000)
    r = Run(wl)
    stats = r.run()
    assert len(r.oracle_log.evlog) > 0, "eviction did not fire"
    report("multiturn small", stats)


def test_decode_small_every_row():
    log("decode small")
    wl = workloads.decode_bf16(n_seq=24, n_prefix=4, prefix_len=256, ctx_range=(300, 1500), steps=3,
                               pool_slots=60000)
    r = Run(wl, check_pool=True)
    stats = r.run()
    assert r.shared_items > 0, "the shared-prefix decode did not run"
    report("decode small", stats)


def test_decode_two_long_sequences_many_splits():
    log("decode two long sequences")
    # two sequences only: the automatic chunk drops to 128 tokens, about 110 splits each
    wl = workloads.decode_bf16(n_seq=2, n_prefix=1, prefix_len=1024, ctx_range=(12000, 15000), steps=2,
                               pool_slots=40000)
    r = Run(wl)
    r.eng.PRIVATE_MAX_WORKGROUPS = 0   # the private tails stay with the split phase
    stats = r.run()
    assert r.shared_items == 8         # one item per shared 128-token chunk of the 1,024-token prefix
    report("decode two long sequences", stats)


def test_longctx_small_every_row():
    log("longctx small")
    wl = workloads.longctx_fp8(prefix_len=2048, suffix_len=200, n_req=4, steps=3, pool_slots=8192)
    r = Run(wl, check_pool=True)
    stats = r.run()
    assert r.shared_items > 0, "the shared-prefix decode did not run"
    report("longctx small", stats)


def test_tot_small_every_row():
    log("tot small")
    # multi-head attention (group size 1) on a branching tree: many template splits, short extends
    wl = workloads.tot_bf16(root_len=200, branching=3, depth=3, thought_range=(10, 40), decode_steps=3,
                            pool_slots=20000)
    stats = Run(wl, check_pool=True).run()
    report("tot small", stats)


# ---------------------------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------------------------

def _edge_workload(qo):
    """Requests with e = 1, p = 0, a full hit (e = 0), a single-token context, ragged tails."""
    shape = workloads.Shape(32, 8, 128, "bf16", "bf16", 1 / math.sqrt(128)) if qo == "bf16" else \
        workloads.Shape(8, 8, 64, "f32", "f32", 1 / 8)
    rng = np.random.default_rng(11)
    b = workloads._Builder(rng, 5000)
    base = b.segment(0, 150)
    lone = b.segment(0, 1)                     # context of one token, no prefix
    reqs_a = [workloads._concat([base])]        # p = 0, e = 150
    reqs_b = [workloads._concat([base, b.segment(base[0], 1)]),        # e = 1
              workloads._concat([base]),                                 # full hit: e = 0
              workloads._concat([lone]),                                 # L = 1
              workloads._concat([base, b.segment(base[0], 129)]),      # ragged tail over tiles
              workloads._concat([base, b.segment(base[0], 33)])]
    vt = workloads.ValueTable(11, b.next_row, shape)
    free = rng.permutation(4096).astype(np.int32)
    return workloads.Workload("edge", 11, shape, 4096, free, [], [reqs_a, reqs_b], True,
                              np.zeros((0, 5), np.int32), np.zeros((0, 5), np.int64), vt)


def _shape_workload(hq, hkv, pool, d=128):
    """A shared 300-token prefix, five suffixes of 1-200 tokens and 3 decode steps for one head
    layout: every group size and kv-head count the kernels dispatch on."""
    shape = workloads.Shape(hq, hkv, d, "bf16", pool, 1 / math.sqrt(d))
    rng = np.random.default_rng(hq * 100 + hkv)
    b = workloads._Builder(rng, 5000)
    pre = b.segment(0, 300)
    reqs = [workloads._concat([pre, b.segment(pre[0], n)]) for n in (1, 37, 64, 129, 200)]
    vt = workloads.ValueTable(hq * 100 + hkv, b.next_row + 3 * len(reqs), shape)
    free = rng.permutation(8192).astype(np.int32)
    dt = rng.integers(0, 5000, size=(3, len(reqs)), dtype=np.int64).astype(np.int32)
    dr = (b.next_row + np.arange(3 * len(reqs), dtype=np.int64)).reshape(3, len(reqs))
    wl = workloads.Workload(f"shape{hq}x{hkv}", 0, shape, 8192, free,
                            [workloads.Request(pre[1].copy(), pre[2].copy(), "prefix")], [reqs], True, dt, dr, vt)
    if pool == "fp8_e4m3":
        wl.k_scale, wl.v_scale = workloads.fp8_scales(vt)
        wl.k_inv_scale = (np.float32(1.0) / wl.k_scale).astype(np.float32)
        wl.v_inv_scale = (np.float32(1.0) / wl.v_scale).astype(np.float32)
    return wl


@pytest.mark.parametrize("hq,hkv,pool", [(32, 16, "bf16"), (16, 16, "bf16"), (16, 8, "bf16"), (32, 32, "fp8_e4m3"),
                                         (16, 2, "bf16"), (32, 4, "fp8_e4m3"), (8, 1, "bf16")])
def test_head_layouts_every_row(hq, hkv, pool):
    log(f"head layout {hq}/{hkv} {pool}")
    stats = Run(_shape_workload(hq, hkv, pool), check_pool=True).run()
    report(f"head layout {hq}/{hkv} {pool}", stats)
    assert {s["kind"] for s in stats} == {"extend", "decode"}


@pytest.mark.parametrize("hq,hkv,pool", [(32, 8, "bf16"), (16, 16, "fp8_e4m3"), (24, 8, "bf16")])
def test_head_dim_64_every_row(hq, hkv, pool):
    """Head dim 64 with bf16 q/o (the VALU extend kernel, the d = 64 split kernels; no
    shared-prefix pass at this head dim), including a group size of 3 for extend."""
    log(f"head dim 64 {hq}/{hkv} {pool}")
    wl = _shape_workload(hq, hkv, pool, d=64)
    if hq // hkv == 3:   # decode takes group sizes 1, 2, 4 and 8 only
        wl.decode_tokens = wl.decode_tokens[:0]
        wl.decode_rows = wl.decode_rows[:0]
    stats = Run(wl, check_pool=True).run()
    report(f"head dim 64 {hq}/{hkv} {pool}", stats)
    kinds = {s["kind"] for s in stats}
    assert "extend" in kinds and (hq // hkv == 3 or "decode" in kinds)


@pytest.mark.parametrize("qo", ["bf16", "f32"])
def test_edge_cases(qo):
    log(f"edge {qo}")
    wl = _edge_workload(qo)
    r = Run(wl)
    stats = r.run()
    assert r.oracle_log.batches[1].extend_lens == [1, 0, 1, 129, 33]
    report(f"edge {qo}", stats)


@pytest.mark.parametrize("pool", ["bf16", "fp8_e4m3"])
def test_pool_beyond_4gib_high_slots(pool):
    """A pool of more than 4 GiB per tensor with the allocator handing out its highest slots
    first: every gathered row lies beyond byte offset 2^32 of its pool, so the gathers must
    address it with 64-bit arithmetic (extend, decode and the shared-prefix decode)."""
    log(f"pool beyond 4 GiB ({pool})")
    if pool == "bf16":
        wl = workloads.fewshot_bf16(n_req=6, prefix_len=300, suffix_range=(40, 200), decode_steps=2)
    else:
        wl = workloads.longctx_fp8(prefix_len=640, suffix_len=150, n_req=4, steps=2, pool_slots=8192)
    row = wl.shape.hkv * wl.shape.d * (2 if pool == "bf16" else 1)
    wl.pool_slots = (1 << 32) // row + 65536                 # 2^32 bytes and then some
    wl.free_order = np.arange(wl.pool_slots - 1, wl.pool_slots - 1 - 40000, -1, dtype=np.int32)
    assert int(wl.free_order.min()) * row >= 1 << 32
    r = Run(wl, check_pool=True)
    stats = r.run()
    assert r.shared_items > 0
    report(f"pool beyond 4 GiB ({pool})", stats)


@pytest.mark.parametrize("private", [False, True], ids=["shared", "private"])
@pytest.mark.parametrize("case", ["longctx", "decode", "fewshot"])
def test_decode_shared_spans(case, private):
    """The shared-prefix pass with items spanning several chunks (a low workgroup target makes
    the plan merge chunks), with and without one-member items over the private tails: every
    decode row against the oracle, both paths."""
    log(f"decode shared spans ({case}, {'private items' if private else 'shared items only'})")
    if case == "longctx":
        wl = workloads.longctx_fp8(prefix_len=2048, suffix_len=200, n_req=4, steps=2, pool_slots=8192)
    elif case == "decode":
        wl = workloads.decode_bf16(n_seq=24, n_prefix=4, prefix_len=512, ctx_range=(600, 1500), steps=2,
                                   pool_slots=60000)
    else:
        wl = workloads.fewshot_bf16(n_req=6, prefix_len=900, suffix_range=(40, 120), decode_steps=2)
    r = Run(wl)
    r.eng.RESIDENT_WORKGROUPS = 16
    r.eng.PRIVATE_MAX_WORKGROUPS = 1 << 20 if private else 0
    stats = r.run()
    assert r.plan is not None and int(r.plan["items"][:, 3].max()) >= 2, "no item spans two chunks"
    skip = r.plan["skip"].cpu().numpy()
    ends = (r.plan_lens + r.plan["chunk"] - 1) // r.plan["chunk"]
    assert np.array_equal(skip, ends) if private else (skip < ends).any()
    report(f"decode shared spans ({case}, private {private})", stats)


def test_decode_split_invariance_and_extend_agreement():
    """Decode over one context with several chunk sizes agrees with itself and with extend's last row."""
    log("decode split invariance")
    wl = workloads.fewshot_bf16(n_req=6, prefix_len=900, suffix_range=(40, 300), decode_steps=0)
    r = Run(wl)
    r.run()
    torch.cuda.synchronize()
    eng = r.eng
    # a second identical batch is a full hit, so its last token can be decoded over the cached context
    reqs = wl.batches[0]
    import prefix_shared_kv_match_amd.runtime as rtm
    hb = eng.prepare([x.tokens[:-1] for x in reqs], r.stride)
    assert hb.extend_lens.tolist() == [0] * len(reqs)
    slots = eng.decode_alloc(hb)
    last_rows = np.array([x.rows[-1] for x in reqs])
    r.scatter(slots, last_rows)
    q = src_tensor(torch, wl.values.q(last_rows), wl.shape, "cuda")
    r2t = torch.from_numpy(hb.req_to_token.copy()).cuda()
    sl = torch.from_numpy(hb.seq_lens.copy()).cuda()
    max_len = int(hb.seq_lens.max())
    outs = []
    for chunk in (64, 128, 256, 1024):
        ws, _ = eng.decode_workspace(hb.n, max_len, chunk)
        outs.append(eng.decode(q, r2t, sl, max_len, ws, chunk).float().cpu().numpy())
        plan = eng.decode_plan(hb.req_to_token, hb.seq_lens, chunk)
        assert plan is not None or chunk > 900          # the 900-token prefix holds no whole 1,024 chunk
        if plan is not None:
            outs.append(eng.decode(q, r2t, sl, max_len, ws, chunk, plan=plan).float().cpu().numpy())
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 * 2.0 ** -8 * np.abs(outs[0]).max()
    ref = np.stack([oa.decode_row(wl, x.rows) for x in reqs])
    compare(outs[0], ref, "bf16", "decode vs oracle")
    eng.release(hb)


# ---------------------------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------------------------

def test_fewshot_full_sampled():
    log("fewshot full")
    stats = Run(workloads.fewshot_bf16(), sample_rows=12).run(decode_sample=16)
    report("fewshot full", stats)


def test_longctx_full_sampled():
    """The long-context case at full size: extend, then all 64 decode steps (sampled sequences
    compared at the first, middle and last step)."""
    log("longctx full")
    stats = Run(workloads.longctx_fp8(), sample_rows=6).run(decode_sample=8)
    assert sorted({s["step"] for s in stats if s["kind"] == "decode"}) == [0, 32, 63]
    report("longctx full", stats)


def test_decode_full_sampled():
    """The decode batch at full size: all 32 steps (sampled sequences compared at the first,
    middle and last step)."""
    log("decode full")
    stats = Run(workloads.decode_bf16()).run(decode_sample=24)
    assert sorted({s["step"] for s in stats if s["kind"] == "decode"}) == [0, 16, 31]
    report("decode full", stats)


def test_multiturn_full_sampled():
    log("multiturn full")
    stats = Run(workloads.multiturn_bf16(), sample_rows=3, req_stride=4).run()
    report("multiturn full", stats)


def test_tot_full_sampled():
    log("tot full")
    stats = Run(workloads.tot_bf16(decode_steps=4), sample_rows=4, req_stride=2).run(decode_sample=32)
    report("tot full", stats)


# ---------------------------------------------------------------------------------------------
# stress: sharp softmax and planted late keys (the running-maximum moves after the first tile)
# ---------------------------------------------------------------------------------------------

def _late_key_fraction(wl, plant_pos, first_tile=64):
    """Host check that the case exercises what it is for: the fraction of (extend query row,
    head) pairs that see a planted key whose logit exceeds the maximum over the first K/V tile
    (positions 0..63) by more than 8 log2 units -- the lazy-rescale threshold of the MFMA
    kernels, so each such row must move its reference maximum and rescale its accumulators."""
    s = wl.shape
    vt = wl.values
    hits = tot = 0
    for r in wl.batches[0]:
        L = len(r.tokens)
        p = L - len(r.rows[300:])
        k = vt.k(r.rows[:L]).astype(np.float64)
        q = vt.q(r.rows[p:L]).astype(np.float64)
        qpos = np.arange(p, L)
        for h in range(s.hq):
            g = h // s.group
            lg = s.sm_scale * (q[:, h] @ k[:, g].T) / math.log(2)      # log2 units
            first = lg[:, :first_tile].max(axis=1)
            fires = np.zeros(qpos.size, dtype=bool)
            for pos in plant_pos(r):
                if pos < L:
                    fires |= (lg[:, pos] - first > 8) & (qpos >= pos)
            hits += int(fires.sum())
            tot += qpos.size
    return hits / tot


@pytest.mark.parametrize("hq,hkv,pool", [(8, 8, "bf16"), (32, 8, "bf16"), (64, 8, "bf16"),
                                         (8, 8, "fp8_e4m3"), (32, 8, "fp8_e4m3"), (64, 8, "fp8_e4m3")])
def test_sharp_softmax_planted_late_keys(hq, hkv, pool):
    """Queries scaled by 4 (a sharp softmax) and two planted keys late in the contexts: one at
    prefix position 200 (the fourth 64-token tile, seen by every extend and decode row, inside
    the second tile of a 128-token shared-prefix decode chunk) and one 100 tokens into the
    longest suffix (seen only by that request's later rows).  Their logits exceed the first
    tile's maximum by more than 8 log2 units for most rows (checked on the host), so the
    extend kernels (group sizes 1, 4, 8; bf16 and fp8 pools), the shared-prefix decode and the
    split phase must all move their running maximum mid-stream.  Every row against the oracle."""
    log(f"sharp softmax, planted keys {hq}/{hkv} {pool}")
    wl = _shape_workload(hq, hkv, pool)
    pre = wl.pre_insert[0].rows
    longest = wl.batches[0][-1]
    wl.values = workloads.StressValues(wl.values, q_mul=4.0, beta=8.0, gamma=60.0,
                                       plant_rows=[int(pre[200]), int(longest.rows[400])])
    if pool == "fp8_e4m3":
        wl.k_scale, wl.v_scale = workloads.fp8_scales(wl.values)
        wl.k_inv_scale = (np.float32(1.0) / wl.k_scale).astype(np.float32)
        wl.v_inv_scale = (np.float32(1.0) / wl.v_scale).astype(np.float32)
    frac = _late_key_fraction(wl, lambda r: [200] + ([400] if r is longest else []))
    assert frac > 0.5, f"only {frac:.2f} of the rows meet a planted key beyond the rescale threshold"
    r = Run(wl, check_pool=True)
    r.eng.RESIDENT_WORKGROUPS = 1 << 20      # one item per chunk: position 200 sits in chunk 1's second tile
    r.eng.PRIVATE_MAX_WORKGROUPS = 0
    stats = r.run()
    assert r.shared_items > 0
    report(f"sharp/planted {hq}/{hkv} {pool} (late-key rows {frac:.2f})", stats)
    assert {s["kind"] for s in stats} == {"extend", "decode"}


# ---------------------------------------------------------------------------------------------
# finished sequences whose decoded tokens another sequence already cached
# ---------------------------------------------------------------------------------------------

def test_finish_duplicates_then_reuse_decoded_tokens():
    """Two sequences with the same prompt decode the same tokens (same K/V rows); a third decodes
    others.  At finish the first one's decoded tokens are inserted with its slots and the second
    one's slots for them are duplicates that go back to the free list (the radix-cache page: the
    caller frees the indices insert reports as already cached).  Host state after finish equals
    the oracle's; then a follow-up request extends the first sequence's full token list and must
    reuse its decoded tokens' slots, whose K/V the decode steps wrote: its extend rows against
    the oracle's attention over the whole context."""
    import prefix_shared_kv_match_amd as pkv
    log("finish duplicates, then reuse of decoded tokens")
    shape = workloads.Shape(32, 8, 128, "bf16", "bf16", 1 / math.sqrt(128))
    rng = np.random.default_rng(21)
    b = workloads._Builder(rng, 5000)
    pre = b.segment(0, 200)
    s1 = b.segment(pre[0], 50)
    s2 = b.segment(pre[0], 70)
    reqs = [workloads._concat([pre, s1]), workloads._concat([pre, s1]), workloads._concat([pre, s2])]
    steps = 3
    dt, dr = workloads._decode(b, 3, steps)
    dt[:, 1], dr[:, 1] = dt[:, 0], dr[:, 0]                     # sequence 1 decodes what sequence 0 decodes
    follow = b.segment(int(dt[-1, 0]) + 1, 40)                  # rows of the follow-up's new tokens
    vt = workloads.ValueTable(21, b.next_row, shape)
    free = rng.permutation(8192).astype(np.int32)
    wl = workloads.Workload("finish_dup", 21, shape, 8192, free,
                            [workloads.Request(pre[1].copy(), pre[2].copy(), "prefix")], [reqs], True, dt, dr, vt)
    r = Run(wl, check_pool=True)
    stats = r.run()
    assert {s["kind"] for s in stats} == {"extend", "decode"}
    ol = r.oracle_log
    eng = r.eng
    assert pkv.rt_dump(eng.tree) == ol.dump
    assert pkv.rt_copy_free_list(eng.tree).tolist() == ol.free
    dup = [ol.decode_slots[s][1] for s in range(steps)]
    assert ol.free[-steps:] == dup                              # sequence 1's decode slots went back
    # follow-up: sequence 0's full token list plus 40 new tokens
    full0 = np.concatenate([reqs[0].tokens, dt[:, 0]])
    rows0 = np.concatenate([reqs[0].rows, dr[:, 0]])
    fr = workloads.Request(np.concatenate([full0, follow[1]]).astype(np.int32),
                           np.concatenate([rows0, follow[2]]).astype(np.int64), "follow-up")
    hb = eng.prepare([fr.tokens], wl.max_len() + 64)
    assert int(hb.prefix_lens[0]) == full0.size
    row0 = ol.batches[0].rows[0] + [ol.decode_slots[s][0] for s in range(steps)]
    assert hb.req_to_token[0, :full0.size].tolist() == row0
    new_rows = fr.rows[full0.size:]
    r.scatter(hb.new_slots, new_rows)
    dtb = eng.device_tables(hb)
    o = eng.extend(dtb, src_tensor(torch, wl.values.q(new_rows), shape, "cuda"))
    torch.cuda.synchronize()
    st = compare(o.float().cpu().numpy(), oa.extend_rows(wl, fr, full0.size), "bf16", "follow-up extend")
    eng.release(hb)
    log(f"finish duplicates: follow-up extend {st}")


def test_kv_scatter_skips_slots_outside_the_pool():
    """A slot list holding -1 and num_slots: those tokens are not written (no write leaves the
    pools), every other token lands bit-exactly, and no other slot changes."""
    import prefix_shared_kv_match_amd as pkv
    log("kv_scatter with slots outside the pool")
    rng = np.random.default_rng(5)
    n, hkv, d, total = 64, 8, 128, 1024
    src = workloads.round_to_bf16(rng.standard_normal((n, hkv, d)).astype(np.float32))
    slots = rng.permutation(total)[:n].astype(np.int32)
    slots[3], slots[40] = -1, total
    kp = torch.zeros((total, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    x = torch.from_numpy(src).to(torch.bfloat16).cuda()
    pkv.pkv_kv_scatter(x, x, torch.from_numpy(slots).cuda(), kp, vp)
    torch.cuda.synchronize()
    good = np.ones(n, dtype=bool)
    good[[3, 40]] = False
    got = kp.cpu()[torch.from_numpy(slots[good].astype(np.int64))].float().numpy()
    np.testing.assert_array_equal(got, src[good])
    mask = np.ones(total, dtype=bool)
    mask[slots[good]] = False
    assert torch.count_nonzero(kp.cpu()[torch.from_numpy(mask)]).item() == 0
    assert torch.count_nonzero(vp.cpu()[torch.from_numpy(mask)]).item() == 0
