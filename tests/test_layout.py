"""Packed-stream geometry (CPU): the unit/batch split of every stage covers each weight tile
exactly once, for the workload shapes and for ragged ones (row lengths of 1, 2, 3, 12 tiles,
stages with fewer pairs than waves, compute-unit counts that do not divide the rows)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "layout_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("layout") / "layout_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "hbm_bandwidth_bound_amd", "csrc"), SRC,
                    "-o", exe], check=True)
    return exe


SHAPES = [
    # L, d, nq, nkv, hd, F, V, max_seq, nwg
    (2, 256, 4, 2, 64, 1024, 4096, 64, 256),          # tiny: 1-tile rows, most waves idle
    (24, 2048, 16, 8, 128, 8192, 32768, 64, 256),     # 1.6B
    (32, 4096, 32, 8, 128, 14336, 128256, 64, 256),   # 8B
    (3, 768, 12, 4, 64, 3072, 5000, 64, 96),          # 3-tile and 12-tile rows, 96 units
    (1, 512, 8, 8, 64, 1536, 1002, 64, 40),           # 2-tile rows, 6-tile F
    # mixture of experts (F is ignored: A x Fe), + E A Fe
    (2, 256, 8, 1, 128, 0, 4096, 64, 256, 16, 4, 256),          # tiny-moe
    (2, 512, 8, 1, 128, 0, 4096, 64, 256, 32, 8, 768),          # small-moe: down units span experts
    (2, 2048, 32, 4, 128, 0, 151936, 64, 256, 128, 8, 768),     # the 128-expert model's layers
    (1, 768, 8, 1, 128, 0, 1000, 64, 40, 6, 3, 512),            # ragged: 3-tile rows, 40 CUs
    # 8-bit weights: tiles of 512 weights of a row
    (2, 512, 8, 4, 64, 1536, 4096, 64, 256, "fp8"),             # tiny-fp8: 1- and 3-tile rows
    (24, 2048, 16, 8, 128, 8192, 32768, 64, 256, "fp8"),        # 1.6B
    (32, 4096, 32, 8, 128, 14336, 128256, 64, 256, "fp8"),      # 8B: 28-tile FFN rows
    (1, 1536, 12, 4, 128, 2560, 1002, 64, 40, "fp8"),           # 3-tile and 5-tile rows, 40 CUs
]


@pytest.mark.parametrize("shape", SHAPES)
def test_units_cover_every_tile_once(checker, shape):
    r = subprocess.run([checker] + [str(x) for x in shape], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout
