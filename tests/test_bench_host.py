"""Host-side parts of bench.py that run without a GPU: the one-GPU refusal
and the reading of the committed HBM-traffic summary."""
import importlib.util
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def _summary():
    text = open(os.path.join(ROOT, "profiles", "hbm_traffic.md")).read()
    start = text.index("```json")
    return json.loads(text[start + 7:text.index("```", start + 7)])


def test_traffic_summary_is_read_as_written():
    b = _bench()
    data = _summary()
    for k, sha in data["source_sha256"].items():
        assert k in b.KERNEL_SOURCES and re.fullmatch(r"[0-9a-f]{64}", sha)
    for w in ("c2", "c3", "c4", "c5"):
        for k in ("block_attn", "unmask_threshold", "kv_refresh"):
            e = data["workloads"][w][k]
            want = int(round(e["fetch_kib"] * 1024 * data["fetch_scale"] + e["write_kib"] * 1024 * data["write_scale"]))
            got = b.measured_traffic(w, k)
            # the counters apply only to the sources they were taken on
            if data["source_sha256"][k] == b.kernel_source_sha256(k):
                assert got == want
            else:
                assert got is None
    assert b.measured_traffic("c2", "no_such_kernel") is None
    assert b.measured_traffic("no_such_workload", "block_attn") is None


def test_traffic_is_near_the_algorithmic_bytes():
    # the summary's HBM bytes per launch against the kernels' algorithmic
    # bytes: the refresh and the unmask move about what they must, the
    # attention partials add a known fraction
    summary = _summary()
    data = summary["workloads"]

    def mb(w, k):
        e = data[w][k]
        return (e["fetch_kib"] * summary["fetch_scale"] + e["write_kib"] * summary["write_scale"]) * 1024 / 1e6

    assert abs(mb("c2", "kv_refresh") / 25.17 - 1) < 0.02
    assert abs(mb("c4", "kv_refresh") / 2684.35 - 1) < 0.02
    assert 1.0 <= mb("c2", "unmask_threshold") / 8.09 < 1.1
    assert 1.0 <= mb("c4", "block_attn") / 1358.95 < 1.02
