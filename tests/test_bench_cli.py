"""bench.py's command-line contract on the CPU: more than one GPU is refused with a message,
every workload has default step counts, and a stored HBM-traffic figure is withheld once the
kernel sources it was measured on have changed."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_default_steps_for_every_workload():
    for wl in ("fewshot_bf16", "decode_bf16", "longctx_fp8", "multiturn_bf16", "tot_bf16"):
        warm, steps = bench.DEFAULT_WARMUP_STEPS[wl]
        assert warm >= 1 and steps >= 1


def test_traffic_withheld_for_changed_sources(monkeypatch):
    key = ("fewshot_bf16", "extend_attention")
    entry = dict(bench.TRAFFIC[key])
    entry["src_hash"] = bench.kernel_src_hash("extend_attention")
    monkeypatch.setitem(bench.TRAFFIC, key, entry)
    got = bench.traffic_bytes(*key)
    assert got == (entry["fetch_kib"] * bench.FETCH_SCALE + entry["write_kib"] * bench.WRITE_SCALE) * 1024.0
    monkeypatch.setitem(bench.TRAFFIC, key, dict(entry, src_hash="0" * 16))
    assert bench.traffic_bytes(*key) is None
    monkeypatch.delitem(bench.TRAFFIC, ("fewshot_bf16", "decode_attention"))
    assert bench.traffic_bytes("fewshot_bf16", "decode_attention") is None     # no figure for that kernel


def test_default_workload_is_the_long_context_case(monkeypatch):
    """With no flags the bench runs the largest configuration that fits one GPU: the long-context
    case (extend over a 32,768-token prefix, then 64 decode steps)."""
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.workload == "longctx_fp8" and a.gpus == 1


def test_cpu_baseline_process_pool():
    """The CPU baseline runs the oracle in a pool of one-thread processes over (request, rows)
    units and reports the tokens done over the longest process's time."""
    import types
    import workloads
    wl = workloads.make("fewshot_bf16")
    hb = types.SimpleNamespace(prefix_lens=np.zeros(len(wl.batches[-1]), dtype=np.int32))
    out = bench.cpu_baseline(wl, {}, hb, 2, min_seconds=0.2, rows_per_req=6, max_workers=3)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s" and out["cores"] == 3
    assert out["value"] > 0 and "3 processes" in out["sample"] and "6 sampled extend rows" in out["sample"]
    dec = bench.cpu_baseline(workloads.make("decode_bf16", steps=2), {"steps": 2}, None, 2, decode_only=True,
                             steps_done=1, min_seconds=0.1, max_workers=2)
    assert dec["cores"] == 2 and dec["value"] > 0 and "newest decode row" in dec["sample"]
