"""The C-ABI library on a machine without a GPU: it loads, exports every function that
include/*.h declares, and its host-side paths fail cleanly (no compute calls are made)."""
import ctypes as C
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from hbm_bandwidth_bound_amd import build, kie
    if not os.path.exists(kie.LIB_PATH):
        build.build()
    return kie.load()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(kie_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_headers_declare_the_entry_points():
    names = declared_functions()
    for n in ("kie_create", "kie_prefill", "kie_decode_step", "kie_generate", "kie_sync", "kie_destroy"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    from hbm_bandwidth_bound_amd import kie
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"
    out = subprocess.run(["nm", "-D", "--defined-only", kie.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\b(kie_\w+)\b", out))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    seen = set()
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        s = lib.kie_status_string(st)
        assert s and s.decode()
        seen.add(s)
    assert len(seen) == 8
    assert lib.kie_status_string(-99)


def test_no_gpu_paths_fail_cleanly(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from hbm_bandwidth_bound_amd import kie, synth
    cfg = kie.make_config(synth.TINY, 96)
    # sizes depend on the device's compute-unit count: 0 without a device
    assert lib.kie_packed_weight_bytes(C.byref(cfg)) == 0
    assert lib.kie_workspace_bytes(C.byref(cfg)) == 0
    assert lib.kie_num_workgroups() <= 0
    assert lib.kie_packed_weight_bytes(None) == 0
    ctx = C.c_void_p()
    st = lib.kie_create(C.byref(cfg), None, None, None, None, None, C.byref(ctx))
    assert st < 0 and not ctx.value
    assert lib.kie_last_error(None)
    # calls on a NULL context are argument errors, not crashes
    assert lib.kie_sync(None) == -1
    assert lib.kie_reset(None) == -1
    assert lib.kie_set_position(None, 0) == -1
    lib.kie_destroy(None)


def test_create_rejects_misaligned_buffers_before_touching_the_device(lib):
    """The KV cache and the workspace must start on a 256-byte boundary (each cache row then owns
    whole cache lines); the check is made before any HIP call, so it holds without a GPU. The
    pointers are never dereferenced."""
    from hbm_bandwidth_bound_amd import kie, synth
    cfg = kie.make_config(synth.TINY, 96)
    w = kie.kie_weights()
    ctx = C.c_void_p()
    base = 1 << 20
    for packed, kv, ws in ((base, base + 16, base), (base, base + 128, base), (base, base, base + 64),
                           (base + 8, base, base)):
        st = lib.kie_create(C.byref(cfg), C.byref(w), C.c_void_p(packed), C.c_void_p(kv), C.c_void_p(ws), None,
                            C.byref(ctx))
        assert st == -1 and not ctx.value  # KIE_ERR_INVALID_ARG
        assert b"256-byte" in lib.kie_last_error(None)


def test_setters_reject_a_null_context(lib):
    assert lib.kie_set_abort_flag(None, None) == -1
    assert lib.kie_set_wait_timeout(None, 5) == -1
    assert lib.kie_set_skew(None, 1) == -1


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without the built library the binding raises instead of computing elsewhere."""
    from hbm_bandwidth_bound_amd import kie
    monkeypatch.setattr(kie, "_lib", None)
    monkeypatch.setattr(kie, "LIB_PATH", str(tmp_path / "absent" / "libkie.so"))
    with pytest.raises(RuntimeError):
        kie.load()
