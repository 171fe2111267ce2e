"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The C oracle (oracle/oracle.c), built with gcc and both sanitizers, runs a tiny dense, an fp8 and
  a mixture-of-experts model plus sampler and router edge cases (tests/native/oracle_sanitize_main.c).
* The decode library's host code (api.cpp and the host side of the kernel units), built with hipcc
  with the sanitizers on the host pass only (each -fsanitize= behind -Xarch_host; the GPU code is
  built as usual), runs its argument checks, size queries and NULL-context calls without a device
  (tests/native/api_sanitize_main.cpp). No kernel is launched.

Any out-of-bounds access, use after free or undefined operation aborts the driver with a report.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(exe, env_extra=None):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"  # the HIP runtime keeps allocations
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    if env_extra:
        env.update(env_extra)
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_oracle_under_asan_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-o", exe,
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(NATIVE, "oracle_sanitize_main.c"),
                    "-lm"], check=True, capture_output=True, text=True)
    r = _run(exe, {"OMP_NUM_THREADS": "1"})
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_library_host_paths_under_asan_ubsan(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the driver checks the paths taken without a device")
    from hbm_bandwidth_bound_amd import build
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc missing")
    flags = [f for f in build.HIPCC_FLAGS if f != "-shared"] + ["-g"] + HOST_SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *flags, "-c", "-o", obj, src], capture_output=True, text=True)
        return obj, r

    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES] + [os.path.join(NATIVE, "api_sanitize_main.cpp")]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(compile_one, srcs))
    for obj, r in results:
        assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "api_san")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *HOST_SAN, "-o", exe] + [o for o, _ in results],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_init" in out and "__ubsan_handle" in out  # the host code is instrumented
    r = _run(exe)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr[-3000:]
