"""Host-side checks of bench.py: the one-GPU contract and the counter-summary reader."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_traffic_summary_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    bench = _bench_module()
    from hbm_bandwidth_bound_amd.build import source_hash
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "steps_per_launch = 64\nhbm_bytes_per_step = 3351511724\n"
    (prof / "traffic_decode_x.txt").write_text(f"source_sha = {source_hash()}\n" + body)
    (prof / "traffic_decode_y.txt").write_text("source_sha = 0000000000000000\n" + body)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("x") == {"bytes_per_step": 3351511724.0, "steps_per_launch": 64}
    assert bench.read_traffic("y") is None  # taken on other sources
    assert bench.read_traffic("z") is None  # no summary


def test_committed_summary_agrees_with_the_byte_model():
    """The algorithmic bytes the counter summary was compared against are those of the byte model
    for the same workload and launch, and the counted bytes are not below them."""
    from hbm_bandwidth_bound_amd import synth, traffic
    path = os.path.join(ROOT, "profiles", "traffic_decode_1.6b-1k.txt")
    if not os.path.exists(path):
        pytest.skip("no counter summary committed")
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    wl = synth.WORKLOADS["1.6b-1k"]
    steps = int(kv["steps_per_launch"])
    algo = traffic.launch_bytes(wl.model, wl.prompt_len, steps) / steps
    assert abs(float(kv["algorithmic_bytes_per_step"]) - algo) <= 1.0
    assert float(kv["hbm_bytes_per_step"]) >= 0.99 * algo


def test_bench_byte_model_is_the_pinned_one():
    """bench.py prices its roofline with hbm_bandwidth_bound_amd/traffic.py; the byte model pinned
    to the pages' closed forms is oracle/bytes_model.py. They must give the same bytes for every
    workload, at every position, and for whole launches."""
    import oracle
    from hbm_bandwidth_bound_amd import synth, traffic
    for name, wl in synth.WORKLOADS.items():
        m = wl.model
        pinned = oracle.bytes_model.decode_step_bytes_8bit if m.weight_format else oracle.bytes_model.decode_step_bytes
        for pos in (0, wl.prompt_len, wl.prompt_len + 255):
            assert traffic.step_bytes(m, pos) == pinned(m, pos), (name, pos)
        n = 17
        assert traffic.launch_bytes(m, wl.prompt_len, n) == sum(pinned(m, wl.prompt_len + s) for s in range(n)), name
