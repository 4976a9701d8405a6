"""bench.py's command-line contract on the CPU: more than one GPU is refused with a message,
every workload has default step counts, and a stored HBM-traffic figure is withheld once the
kernel sources it was measured on have changed."""
import os
import subprocess
import sys

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
