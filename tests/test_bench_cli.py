"""bench.py's command-line contract and its bookkeeping, on the CPU (no GPU
work is started by any of these)."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = run_bench("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bad_step_counts_are_rejected():
    assert run_bench("--steps", "0").returncode == 2
    assert run_bench("--warmup", "-1").returncode == 2


def test_traffic_entry_is_used_only_for_the_matching_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    traffic = tmp_path / "traffic.json"
    traffic.write_text(json.dumps({"entries": {"w": {"source_sha256": sha, "hbm_bytes_per_launch": 123}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    assert bench.measured_traffic("w", str(src)) == 123
    assert bench.measured_traffic("other", str(src)) is None
    src.write_text("// kernel, changed\n")
    assert bench.measured_traffic("w", str(src)) is None


def test_committed_traffic_entries_name_their_sources():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert rec["entries"], "no traffic entries"
    for name, e in rec["entries"].items():
        assert os.path.exists(os.path.join(ROOT, e["source"])), name
        assert e["hbm_bytes_per_launch"] > 0 and e["algorithmic_bytes"] > 0, name


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_inputs_provenance_matches_committed_digests():
    from attention_attn_fwd_08_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["B1-H1-N256-d64"]
    q, k, v = workload_inputs(w)
    rec = bench.inputs_provenance(w.name, {"q": q, "k": k, "v": v})
    assert rec["inputs_match_committed_digests"] is True
    assert rec["inputs_sha256"]["q"] == hashlib.sha256(q.tobytes()).hexdigest()
    assert set(rec["kernel_sources_sha256"]) == {"attn_fwd.hip", "attn_bwd.hip"}
    # A changed buffer (one bf16 value) no longer matches; an unknown workload has no digests.
    q2 = q.copy()
    q2.flat[7] ^= 1
    assert bench.inputs_provenance(w.name, {"q": q2, "k": k, "v": v})["inputs_match_committed_digests"] is False
    assert bench.inputs_provenance("no-such-workload", {"q": q})["inputs_match_committed_digests"] is None
