"""The exchange protocol of the decode kernel, modelled on the CPU with threads and random delays
(tests/native/exchange_model.cpp): per-layer, per-hop buffers of tagged words with one tag per
step never hand a reader a wrong value and every wait ends. Sharing one buffer across layers, or
reusing one tag across steps, must be caught by the same model."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "exchange_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("exchange") / "exchange_model")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", SRC, "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("threads,layers,steps,seed", [(16, 3, 40, 1), (32, 2, 30, 2), (7, 4, 25, 3)])
def test_protocol_holds_under_random_delays(model, threads, layers, steps, seed):
    r = subprocess.run([model, str(threads), str(layers), str(steps), str(seed)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout


@pytest.mark.parametrize("mode", ["shared", "sametag"])
def test_model_catches_a_broken_layout(model, mode):
    r = subprocess.run([model, "16", "3", "40", "5", mode], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and r.stdout.startswith("FAIL"), r.stdout
