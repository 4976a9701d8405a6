"""GPU parity of the serve-loop paths: cache-aware scheduling (fcfs / lpm over the multi-turn
workload, with eviction) and chunked prefill (launches capped at a token budget).  Host tables
must equal the oracle scheduler's bit-exactly; every extend row is compared with the oracle's
attention over the request's full context (bf16: max|d| <= 2e-2, relative RMS <= 5e-3)."""
import numpy as np
import pytest

import workloads
from oracle import attention as oa
from oracle import driver as od
from oracle import scheduler as osch
from oracle.radix_tree import OracleTree

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from tests.gpu_harness import compare, log, make_engine, src_tensor  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import prefix_shared_kv_match_amd as pkv
    pkv.lib()


def _extend_and_check(eng, wl, reqs, ends, hb, what):
    """Scatter the launch's new K/V, run extend, compare every row with the oracle."""
    new_rows = np.concatenate([reqs[k].rows[int(hb.prefix_lens[k]):e] for k, e in enumerate(ends)]) \
        if hb.n_new else np.zeros(0, dtype=np.int64)
    assert new_rows.size == hb.n_new
    if not hb.n_new:
        return None
    sl = torch.from_numpy(np.ascontiguousarray(hb.new_slots, dtype=np.int32)).cuda()
    eng.scatter(sl, src_tensor(torch, wl.values.k(new_rows), wl.shape, "cuda"),
                src_tensor(torch, wl.values.v(new_rows), wl.shape, "cuda"))
    dt = eng.device_tables(hb)
    o = eng.extend(dt, src_tensor(torch, wl.values.q(new_rows), wl.shape, "cuda"))
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    ref = []
    for k, e in enumerate(ends):
        p = int(hb.prefix_lens[k])
        if e > p:
            ref.append(oa.extend_rows(wl, reqs[k], p, sample=np.arange(p, e)))
    return compare(got, np.concatenate(ref), wl.shape.qo_dtype, what)


SERVE_CASES = [("fcfs", "lru"), ("lpm", "lru"), ("lpm", "lfu"), ("lpm", "slru"), ("lpm", "fifo"), ("lpm", "mru"),
               ("lpm", "filo"), ("lpm", "priority")]


@pytest.mark.parametrize("order,policy", SERVE_CASES)
def test_serve_multiturn_small(order, policy):
    """The serve loop over the multi-turn workload with eviction, under every eviction policy of
    the radix-cache page's strategy list: the policy decides which rows are evicted and so which
    slots later batches reuse and which they refill, i.e. the tables the kernels read.  Picks and
    tables bit-exact against the oracle scheduler with the same policy; every extend row against
    the oracle's attention."""
    from prefix_shared_kv_match_amd import runtime
    log(f"serve multiturn small {order} {policy}")
    wl = workloads.multiturn_bf16(n_conv=24, turns=4, turn_range=(16, 96), batch=8, pool_slots=20000,
                                  capacity=8000)
    arr = [r for b in wl.batches for r in b]
    after = [r.after for r in arr]
    prio = [r.priority for r in arr]
    otree = OracleTree(wl.pool_slots, wl.free_order, policy)
    olog = osch.serve(otree, [r.tokens.tolist() for r in arr], after, order, batch=6, window=24, priorities=prio)
    assert otree.evlog, "eviction did not fire"
    eng = make_engine(wl, policy=policy)
    stats = []

    def on_batch(pick, hb):
        k = len(stats)
        assert pick == olog.picks[k]
        assert hb.prefix_lens.tolist() == olog.tables[k].prefix_lens
        assert hb.new_slots.tolist() == olog.tables[k].new_slots
        reqs = [arr[i] for i in pick]
        stats.append(_extend_and_check(eng, wl, reqs, [len(r.tokens) for r in reqs], hb, f"round {k}"))

    runtime.serve(eng.tree, [r.tokens for r in arr], after, order, 6, 24, wl.max_len(), priorities=prio,
                  on_batch=on_batch)
    assert len(stats) == len(olog.picks)
    log(f"  {len(stats)} rounds, hit rate {olog.hit_rate:.3f}, worst {max(s['rel_rms'] for s in stats if s)}")


@pytest.mark.parametrize("budget", [64, 200, 1000])
def test_chunked_prefill_fewshot_small(budget):
    from prefix_shared_kv_match_amd import runtime
    log(f"chunked prefill budget {budget}")
    wl = workloads.fewshot_bf16(n_req=8, prefix_len=300, suffix_range=(20, 200), decode_steps=0)
    reqs = wl.batches[0]
    o = OracleTree(wl.pool_slots, wl.free_order)
    for r in wl.pre_insert:
        od.release(o, od.prepare_batch(o, [r.tokens]).last_nodes)
    launches = osch.chunked_prefill(o, [r.tokens.tolist() for r in reqs], budget)
    eng = make_engine(wl)
    for r in wl.pre_insert:
        hb = eng.prepare([r.tokens], wl.max_len())
        sl = torch.from_numpy(hb.new_slots.astype(np.int32)).cuda()
        eng.scatter(sl, src_tensor(torch, wl.values.k(r.rows), wl.shape, "cuda"),
                    src_tensor(torch, wl.values.v(r.rows), wl.shape, "cuda"))
        eng.release(hb)
    stats = []

    def on_launch(idx, ends, hb):
        k = len(stats)
        assert (idx, ends) == (launches[k].reqs, launches[k].ends)
        assert hb.prefix_lens.tolist() == launches[k].tables.prefix_lens
        assert hb.new_slots.tolist() == launches[k].tables.new_slots
        assert int(hb.extend_lens.sum()) <= budget
        stats.append(_extend_and_check(eng, wl, [reqs[i] for i in idx], ends, hb, f"launch {k}"))

    runtime.chunked_prefill(eng.tree, [r.tokens for r in reqs], budget, wl.max_len(), on_launch=on_launch)
    assert len(stats) == len(launches) >= (1 if budget >= 1000 else 2)
    log(f"  {len(stats)} launches, worst {max(s['rel_rms'] for s in stats if s)}")


def test_staged_tables_match_plain_upload():
    """The packed, double-buffered table upload the bench and the job loops use gives the same
    extend output as a plain upload, over three consecutive batches (both staging buffers and
    the reuse of the device pack)."""
    log("staged tables")
    wl = workloads.multiturn_bf16(n_conv=12, turns=3, turn_range=(16, 80), batch=6, pool_slots=20000,
                                  capacity=12000)
    eng = make_engine(wl)
    for bi, batch in enumerate(wl.batches[:3]):
        hb = eng.prepare([r.tokens for r in batch], wl.max_len())
        rows = np.concatenate([r.rows[p:] for r, p in zip(batch, hb.prefix_lens)])
        sl = torch.from_numpy(np.ascontiguousarray(hb.new_slots, dtype=np.int32)).cuda()
        eng.scatter(sl, src_tensor(torch, wl.values.k(rows), wl.shape, "cuda"),
                    src_tensor(torch, wl.values.v(rows), wl.shape, "cuda"))
        q = src_tensor(torch, wl.values.q(rows), wl.shape, "cuda")
        plain = eng.extend(eng.device_tables(hb), q)
        staged_tables = eng.device_tables(hb, staged=True)
        for k, v in eng.device_tables(hb).items():
            assert torch.equal(staged_tables[k].cpu(), v.cpu()), (bi, k)
        staged = eng.extend(staged_tables, q)
        torch.cuda.synchronize()
        assert torch.equal(plain, staged), bi
        eng.release(hb)


def test_prepare_staged_rows_upload_like_plain_tables():
    """Slot rows written by prepare_staged straight into the pinned upload buffer give the
    same device tables (over each row's length) and the same extend output as prepare plus a
    plain upload, over three consecutive batches (both staging buffers, buffer reuse)."""
    log("prepare_staged")
    wl = workloads.multiturn_bf16(n_conv=12, turns=3, turn_range=(16, 80), batch=6, pool_slots=20000,
                                  capacity=12000)
    eng = make_engine(wl)
    twin = make_engine(wl)
    for bi, batch in enumerate(wl.batches[:3]):
        toks = [r.tokens for r in batch]
        hs = eng.prepare_staged(toks, wl.max_len())
        hp = twin.prepare(toks, wl.max_len())
        assert hs.prefix_lens.tolist() == hp.prefix_lens.tolist() and hs.new_slots.tolist() == hp.new_slots.tolist()
        rows = np.concatenate([r.rows[p:] for r, p in zip(batch, hp.prefix_lens)])
        for e in (eng, twin):
            h = hs if e is eng else hp
            sl = torch.from_numpy(np.ascontiguousarray(h.new_slots, dtype=np.int32)).cuda()
            e.scatter(sl, src_tensor(torch, wl.values.k(rows), wl.shape, "cuda"),
                      src_tensor(torch, wl.values.v(rows), wl.shape, "cuda"))
        q = src_tensor(torch, wl.values.q(rows), wl.shape, "cuda")
        ds, dp = eng.device_tables(hs, staged=True), twin.device_tables(hp)
        for i, r in enumerate(batch):
            n = len(r.tokens)
            assert torch.equal(ds["req_to_token"][i, :n].cpu(), dp["req_to_token"][i, :n].cpu()), (bi, i)
        a, b = eng.extend(ds, q), twin.extend(dp, q)
        torch.cuda.synchronize()
        assert torch.equal(a, b), bi
        eng.release(hs)
        twin.release(hp)



@pytest.mark.parametrize("side_min_bytes", [0, None])
def test_staged_uploads_queued_without_host_sync(side_min_bytes):
    """Twelve staged table uploads over three batches and eight decode uploads queued
    back-to-back with no host synchronisation: the side-stream copies may run ahead of the
    kernels reading earlier uploads, and every kernel must still see its own tables (extend
    outputs bit-equal to the plain-upload ones; decode slots / lengths read back intact).
    side_min_bytes 0 sends every table on the side stream; None keeps the size rule (these
    small tables then go on the launch stream)."""
    log(f"staged uploads queued without host sync (side stream from {side_min_bytes} bytes)")
    wl = workloads.multiturn_bf16(n_conv=12, turns=3, turn_range=(16, 80), batch=6, pool_slots=20000,
                                  capacity=12000)
    eng = make_engine(wl)
    if side_min_bytes is not None:
        eng._uploader("_tables_up").SIDE_MIN_BYTES = side_min_bytes
    hbs, qs, refs = [], [], []
    for batch in wl.batches[:3]:
        hb = eng.prepare([r.tokens for r in batch], wl.max_len())
        rows = np.concatenate([r.rows[p:] for r, p in zip(batch, hb.prefix_lens)])
        sl = torch.from_numpy(np.ascontiguousarray(hb.new_slots, dtype=np.int32)).cuda()
        eng.scatter(sl, src_tensor(torch, wl.values.k(rows), wl.shape, "cuda"),
                    src_tensor(torch, wl.values.v(rows), wl.shape, "cuda"))
        q = src_tensor(torch, wl.values.q(rows), wl.shape, "cuda")
        refs.append(eng.extend(eng.device_tables(hb), q))
        hbs.append(hb)
        qs.append(q)
    torch.cuda.synchronize()
    outs = []
    for rep in range(4):
        for k in range(3):
            outs.append((k, eng.extend(eng.device_tables(hbs[k], staged=True), qs[k])))
    rng = np.random.default_rng(5)
    dec = []
    for i in range(8):
        s = rng.integers(0, 1 << 20, size=37).astype(np.int32)
        n = rng.integers(1, 4000, size=37).astype(np.int32)
        sd, nd = eng.upload_decode(s, n)
        dec.append((s, n, torch.stack([sd * 1, nd * 1])))    # read on the current stream
    torch.cuda.synchronize()
    for k, o in outs:
        assert torch.equal(o, refs[k]), k
    for s, n, got in dec:
        g = got.cpu().numpy()
        assert np.array_equal(g[0], s) and np.array_equal(g[1], n)
    for hb in hbs:
        eng.release(hb)


def test_decode_shared_identical_and_boundary_contexts():
    """Shared-prefix decode on contexts built to hit the plan's edges: two identical requests
    (a full hit: they share every whole chunk but the newest token's), a context of exactly two
    chunks, one cut inside a shared chunk, one shorter than a chunk, one private, one that
    fills two chunks and then grows into a third; every row equals the plain decode's within
    float32 summation order, and both equal the float64 oracle's attention over each
    sequence's gathered K/V rows (bf16 tolerances).  Both plans: shared chunks only, and with
    the private tails as one-member items (made at the first step and kept while the
    sequences grow, the split phase launched from the first chunk a sequence still needs at
    that step, or not at all)."""
    from prefix_shared_kv_match_amd.runtime import Engine
    log("decode shared: identical and boundary contexts")
    rng = np.random.default_rng(11)
    hq, hkv, d, chunk = 32, 8, 128, 128
    eng = Engine(4096, hq, hkv, d, "bf16", "bf16", None, "cuda")
    base = rng.integers(0, 50_000, size=400).astype(np.int32)
    other = rng.integers(50_000, 100_000, size=400).astype(np.int32)
    reqs = [base[:300], base[:300], base[:256], base[:200], base[:100],
            np.concatenate([base[:128], other[:150]]), other[:333], base[:255]]
    stride = 512
    hb = eng.prepare(reqs, stride)
    n_new = hb.n_new
    k = torch.randn(n_new, hkv, d).to(torch.bfloat16)
    v = torch.randn(n_new, hkv, d).to(torch.bfloat16)
    # host copies of what each slot holds, for the oracle
    kh = np.zeros((4096, hkv, d), dtype=np.float64)
    vh = np.zeros((4096, hkv, d), dtype=np.float64)
    kh[hb.new_slots] = k.float().numpy()
    vh[hb.new_slots] = v.float().numpy()
    eng.scatter(torch.from_numpy(hb.new_slots.astype(np.int32)).cuda(), k.cuda(), v.cuda())
    b = hb.n
    max_len = int(hb.seq_lens.max()) + 3
    ws, _ = eng.decode_workspace(b, max_len, chunk)
    plans = {}
    for step in range(3):
        slots = eng.decode_alloc(hb)
        kn, vn = torch.randn(b, hkv, d).to(torch.bfloat16), torch.randn(b, hkv, d).to(torch.bfloat16)
        kh[slots], vh[slots] = kn.float().numpy(), vn.float().numpy()
        eng.scatter(torch.from_numpy(slots).cuda(), kn.cuda(), vn.cuda())
        qh = torch.randn(b, hq, d).to(torch.bfloat16)
        q = qh.cuda()
        r2t = torch.from_numpy(np.ascontiguousarray(hb.req_to_token)).cuda()
        sl = torch.from_numpy(hb.seq_lens.copy()).cuda()
        if step == 0:
            eng.PRIVATE_MAX_WORKGROUPS = 0
            plans["shared"] = eng.decode_plan(hb.req_to_token, hb.seq_lens, chunk, upload=False)
            eng.PRIVATE_MAX_WORKGROUPS = Engine.PRIVATE_MAX_WORKGROUPS
            plans["private"] = eng.decode_plan(hb.req_to_token, hb.seq_lens, chunk, upload=False)
            # 0, 1 identical (301 tokens: chunks 0, 1 whole and shared); 2 (257) shares both; 3
            # (201) shares chunk 0 only; 4 (101) holds no whole chunk; 5 shares chunk 0 (its own
            # 128 tokens); 6 is private; 7 (256: its newest token ends chunk 1) shares chunk 0
            assert plans["shared"]["skip"].tolist() == [2, 2, 2, 1, 0, 1, 0, 1]
            assert plans["private"]["skip"].tolist() == [3, 3, 3, 2, 1, 3, 3, 2]
            # the same private plan on the device, made once: at this step its items cover every
            # context; at later steps decode() starts the split phase from the lengths it is given
            device_plan = eng.decode_plan(hb.req_to_token, hb.seq_lens, chunk)
            assert device_plan["first_split"] == Engine.NO_SPLIT_PHASE
        plain = eng.decode(q, r2t, sl, max_len, ws, chunk).float()
        shared = eng.decode(q, r2t, sl, max_len, ws, chunk, plan=device_plan, seq_lens_host=hb.seq_lens).float()
        torch.cuda.synchronize()
        diff = (plain - shared).abs().max().item()
        assert diff <= 2.0 ** -7 * plain.abs().max().item(), (step, "device plan", diff)
        # the float64 oracle over each sequence's gathered rows (position L - 1 sees 0..L-1)
        ref = np.stack([oa.attend(qh[i:i + 1].float().numpy(), kh[hb.req_to_token[i, :hb.seq_lens[i]]],
                                  vh[hb.req_to_token[i, :hb.seq_lens[i]]], [hb.seq_lens[i] - 1], 1.0 / np.sqrt(d))[0]
                        for i in range(b)])
        compare(plain.cpu().numpy(), ref, "bf16", f"boundary decode step {step} (plain)")
        compare(shared.cpu().numpy(), ref, "bf16", f"boundary decode step {step} (device plan)")
        for name, host_plan in plans.items():
            _, _, plan = eng.upload_decode(slots, hb.seq_lens, host_plan)
            if name == "private":
                # every chunk is an item at the first step; then sequence 7 grows into chunk 2
                assert plan["first_split"] == (Engine.NO_SPLIT_PHASE if step == 0 else 2), (step, plan["first_split"])
            shared = eng.decode(q, r2t, sl, max_len, ws, chunk, plan=plan).float()
            torch.cuda.synchronize()
            diff = (plain - shared).abs().max().item()
            assert diff <= 2.0 ** -7 * plain.abs().max().item(), (step, name, diff)
    eng.release(hb)
