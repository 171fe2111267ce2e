#!/usr/bin/env python3
"""HBM traffic of one decode launch from rocprofv3 hardware counters.

Two steps:

* ``run`` is the profiled program: the prompt pass (or, with ``--synthetic-kv``, seeded cache rows
  in its place), one ``kie_generate`` launch of ``--steps``
  tokens (the decode kernel dispatch that is measured), then one plain copy of ``--copy-mib`` MiB
  (``stream_copy_kernel``: reads and writes exactly that many bytes), the calibration dispatch.
  It is run twice under ``rocprofv3 --pmc``, once with ``FETCH_SIZE`` and once with
  ``WRITE_SIZE`` (one counter group per pass).
* ``summarize`` reads the two counter CSVs, scales each counter of the decode dispatch by what the
  same counter reads for the copy of known size (bytes per counted KiB), and writes the summary
  that ``bench.py`` reports as ``roofline.traffic``. The summary records the hash of the kernel
  sources it was taken on; ``bench.py`` ignores it once the sources change.

Example (on a machine with the GPU; each pass its own run):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d prof/pmc_fetch -o run -- \\
        python3 -m hbm_bandwidth_bound_amd.traffic_profile run --workload 1.6b-1k --steps 64
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d prof/pmc_write -o run -- \\
        python3 -m hbm_bandwidth_bound_amd.traffic_profile run --workload 1.6b-1k --steps 64
    python3 -m hbm_bandwidth_bound_amd.traffic_profile summarize --workload 1.6b-1k --steps 64 \\
        --fetch prof/pmc_fetch --write prof/pmc_write --out profiles/traffic_decode_1.6b-1k.txt
"""
import argparse
import collections
import csv
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DECODE_KERNEL = "kie_decode_kernel"          # dense layers
MOE_DECODE_KERNEL = "kie_moe_decode_kernel"  # mixture-of-experts layers
FP8_DECODE_KERNEL = "kie_fp8_decode_kernel"  # 8-bit weights
COPY_KERNEL = "stream_copy_kernel"


def decode_kernel(model) -> str:
    if model.n_experts:
        return MOE_DECODE_KERNEL
    return FP8_DECODE_KERNEL if getattr(model, "weight_format", 0) else DECODE_KERNEL


def run(args):
    import torch

    from hbm_bandwidth_bound_amd import synth
    from hbm_bandwidth_bound_amd.kie import Engine, stream_copy

    wl = synth.WORKLOADS[args.workload]
    m = wl.model
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    w = synth.make_weights_torch(m, wl.weight_seed, device=dev)
    P, K = wl.prompt_len, args.steps
    eng = Engine(m, w, P + K)
    prompt = torch.tensor(synth.prompt_ids(P, m.vocab_size, wl.prompt_seed), dtype=torch.int32, device=dev)
    if args.synthetic_kv:
        # the decode launch reads the same bytes whatever the cached rows hold: seeded bf16 rows of
        # about the prompt's magnitude stand in for them, so that the profiled program has no
        # prompt pass (tens of thousands of dispatches at long context)
        g = torch.Generator(device=dev).manual_seed(wl.prompt_seed)
        rows = torch.randn(eng.kv.numel(), generator=g, device=dev, dtype=torch.float32) * 0.5
        eng.kv.copy_(rows.to(torch.bfloat16).view(torch.int16))
        del rows
        eng.set_position(P)
        first = prompt[-1:].clone()
    else:
        first = eng.prefill(prompt)
    eng.sync()
    out = torch.empty(K, dtype=torch.int32, device=dev)
    eng.generate(first, K, out)
    eng.sync()
    nb = args.copy_mib << 20
    src = torch.ones(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    stream_copy(dst, src, nb, stream)
    torch.cuda.synchronize()
    print("done", out[:4].tolist(), flush=True)
    # explicit teardown before the interpreter exits: the context, every device tensor, then the
    # stream, so that nothing of the GPU runtime is released by exit handlers
    eng.close()
    del eng, w, prompt, first, out, src, dst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _counter_per_dispatch(run_dir: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter; a counter reported per hardware
    instance is summed over its instances."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    agg = collections.OrderedDict()
    names = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (f, r["Dispatch_Id"])
                agg[key] = agg.get(key, 0.0) + float(r["Counter_Value"])
                names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in agg.items():
        out[names[key]].append(v)
    return out


def _pick(per_kernel, needle):
    vals = [v for name, vs in per_kernel.items() if needle in name for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of {needle} in the counter output")
    return vals


def summarize(args):
    from hbm_bandwidth_bound_amd import synth, traffic
    from hbm_bandwidth_bound_amd.build import source_hash

    wl = synth.WORKLOADS[args.workload]
    nb = args.copy_mib << 20
    lines = []
    per = {}
    for counter, run_dir in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        d = _counter_per_dispatch(run_dir, counter)
        dec = _pick(d, decode_kernel(wl.model))
        cpy = _pick(d, COPY_KERNEL)
        if len(dec) != 1 or len(cpy) != 1:
            raise SystemExit(f"{counter}: expected one decode and one copy dispatch, got {len(dec)} and {len(cpy)}")
        scale = nb / cpy[0]  # bytes per counted unit (the counters count KiB)
        per[counter] = dec[0] * scale
        lines.append(f"# {counter}: decode dispatch {dec[0]:.6g}, copy of {nb} B {cpy[0]:.6g} "
                     f"-> {scale:.6g} B per unit (nominal 1024)")
    K = args.steps
    algo = traffic.launch_bytes(wl.model, wl.prompt_len, K)
    total = per["FETCH_SIZE"] + per["WRITE_SIZE"]
    with open(args.out, "w") as f:
        f.write(f"# HBM traffic of one {decode_kernel(wl.model)} dispatch ({wl.name}: prompt {wl.prompt_len}, "
                f"{K} decode steps in one launch)\n")
        f.write("# commands (from the repository root, each pass its own run):\n")
        filt = f"--kernel-include-regex '{args.kernel_regex}' " if args.kernel_regex else ""
        syn = " --synthetic-kv" if args.synthetic_kv else ""
        for c, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
            f.write(f"#   rocprofv3 --pmc {c} {filt}--output-format csv -d {d} -o run -- python3 -m "
                    f"hbm_bandwidth_bound_amd.traffic_profile run --workload {wl.name} --steps {K} "
                    f"--copy-mib {args.copy_mib}{syn}\n")
        f.write(f"#   python3 -m hbm_bandwidth_bound_amd.traffic_profile summarize --workload {wl.name} "
                f"--steps {K} --copy-mib {args.copy_mib}{syn} --fetch {args.fetch} --write {args.write} --out {args.out}"
                + (f" --kernel-regex '{args.kernel_regex}'" if args.kernel_regex else "") + "\n")
        for ln in lines:
            f.write(ln + "\n")
        f.write(f"source_sha = {source_hash()}\n")
        f.write(f"steps_per_launch = {K}\n")
        f.write(f"fetch_bytes_per_launch = {per['FETCH_SIZE']:.0f}\n")
        f.write(f"write_bytes_per_launch = {per['WRITE_SIZE']:.0f}\n")
        f.write(f"hbm_bytes_per_step = {total / K:.0f}\n")
        f.write(f"algorithmic_bytes_per_step = {algo / K:.0f}\n")
        f.write(f"traffic_over_algorithmic = {total / algo:.4f}\n")
    print(open(args.out).read())


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("run", "summarize"):
        p = sub.add_parser(name)
        p.add_argument("--workload", default="1.6b-1k")
        p.add_argument("--steps", type=int, default=64)
        p.add_argument("--copy-mib", type=int, default=1024)
        p.add_argument("--synthetic-kv", action="store_true",
                       help="no prompt pass: seeded rows stand in for the cached K/V of the prompt")
        if name == "summarize":
            p.add_argument("--fetch", required=True)
            p.add_argument("--write", required=True)
            p.add_argument("--out", required=True)
            p.add_argument("--kernel-regex", default=None,
                           help="the --kernel-include-regex the counter passes ran with (recorded only)")
    args = ap.parse_args()
    (run if args.cmd == "run" else summarize)(args)


if __name__ == "__main__":
    main()
