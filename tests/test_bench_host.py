"""Host-side pieces of bench.py (no GPU): the byte model, the multi-GPU refusal and
the counter-derived traffic record with its source-hash guard."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_algorithmic_bytes_zipf():
    wl = synth.WORKLOADS["zipf"]
    b = bench.algorithmic_bytes(wl)
    T, H, k, E = 4096, 2048, 6, 64
    assert b["expert"] == 2 * T * k * H * 2
    assert b["dispatch_copy"] == T * H * 2 + T * k * H * 2 + 4 * T * k
    assert b["combine"] == T * k * H * 2 + 8 * T * k + T * H * 2
    assert b["route"] == T * E * 4 + T * k * 8
    assert bench.ffn_flops(synth.WORKLOADS["local_layer"]) == 6 * 8192 * 2 * 4096 * 1408


def test_multi_gpu_request_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err


def test_stored_traffic_record_and_guard(tmp_path, monkeypatch):
    got = bench.stored_traffic("zipf", "expert_scale_kernel")
    if got is not None:  # the record matches the current sources
        assert abs(got - 2 * 4096 * 6 * 2048 * 2) / got < 0.01
    assert bench.stored_traffic("zipf", "no_such_kernel") is None
    fake = tmp_path / "t.md"
    fake.write_text("scale fetch=2.0 write=1.0\n"
                    "traffic workload=zipf kernel=expert_scale_kernel fetch_kib=10 write_kib=20 "
                    "sources=expert.hip code_sha256=0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(fake))
    assert bench.stored_traffic("zipf", "expert_scale_kernel") is None  # sources changed
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.stored_traffic("zipf", "expert_scale_kernel") is None


def test_source_code_hash_ignores_comments_only():
    a = "int f(int x) {  // add one\n  return x + 1; /* done */ }\n"
    b = "// a header comment\nint f(int x) {\n  return x + 1;\n}\n"
    assert bench.source_code_hash(a) == bench.source_code_hash(b)
    assert bench.source_code_hash(a) != bench.source_code_hash(a.replace("x + 1", "x + 2"))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_byte_model_positive(name):
    b = bench.algorithmic_bytes(synth.WORKLOADS[name])
    assert all(v > 0 for v in b.values())


def test_median_of_steps():
    steps = [{"a": 1.0, "b": 2.0}, {"a": 5.0, "b": 0.0}, {"a": 2.0, "b": 2.0}]
    # per-step sums of a + b: 3, 5, 4 -> median 4
    assert bench.StepRunner.median_of(steps, ("a", "b")) == 4.0
    # even count: mean of the middle two (a alone: 1, 2, 5, 7 -> 3.5)
    steps.append({"a": 7.0, "b": 0.0})
    assert bench.StepRunner.median_of(steps, ("a",)) == 3.5
