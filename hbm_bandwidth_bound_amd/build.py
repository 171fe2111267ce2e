"""Build the HIP library (libkie.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkie.so")
SOURCES = ["api.cpp", "monokernel.hip", "kernels_hd64.hip", "kernels_hd128.hip", "kernels_moe.hip", "kernels_fp8.hip", "pack.hip",
           "prefill.hip", "exchange_probe.hip"]

# Packed fp32 instructions are disabled: the compiler may not form v_pk_* f32 ops from float code.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def source_hash() -> str:
    """Short hash of the sources the decode kernel is built from (every file of csrc except the
    prompt pass): a counter summary of that kernel is only used for the sources it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.startswith("prefill."):
            continue
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    """Compile every source to an object in parallel (the two kernel units dominate), then link."""
    from concurrent.futures import ThreadPoolExecutor
    import tempfile
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    tmpdir = tempfile.mkdtemp(prefix="kie_build_")

    def compile_one(src):
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *flags, *extra, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    msgs = []
    failed = False
    for obj, r in results:
        # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
        msgs += [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        failed |= r.returncode != 0
    if failed:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed to compile the decode library")
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to link the decode library")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    for o, _ in results:
        os.remove(o)
    os.rmdir(tmpdir)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
