#!/usr/bin/env python3
"""Per-hop latency and skew of the decode kernel, from a build that stamps its hop timeline.

A decode step crosses six inter-workgroup exchanges per layer (queries/keys/values to attention,
attention partials to the merge, the merged output to every workgroup, then the three gathers of
the residual stream and the FFN activations). A build with -DKIE_TRACE_HOPS takes s_memrealtime
stamps (10 ns) of wave 0 of every workgroup at each exchange of one sampled (step, layer) and of
each weight batch of that layer, and copies them to the workspace when the launch ends.

    python3 -m hbm_bandwidth_bound_amd.hop_profile build         # CPU: libkie_hops.so beside libkie.so
    python3 -m hbm_bandwidth_bound_amd.hop_profile run --workload 1.6b-1k --out profiles/hops_1.6b-1k.md

The report gives, per event, the spread over workgroups; per exchange, the publication spread
(skew) and the time from the last publication to each workgroup holding the gathered words (mean
per chiplet, min, max, and a histogram); the stage durations; the attention phases; and wave 0's
weight batches. The traced build runs the same code with the stamps added.
"""
import argparse
import ctypes as C
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
HOPS_LIB = os.path.join(HERE, "libkie_hops.so")

# stamp slots, in the order of the kernel's HopEvent
EVENTS = ["QKV_IN", "QKV_PUB", "ATT_IN", "ATT_PUB", "MERGE_PUB", "O_GOT", "O_IN", "XA_PUB", "XA_GOT", "GU_IN",
          "H_PUB", "H_GOT", "DN_IN", "XF_PUB", "XF_GOT", "NORM_DONE", "ATT_ALLQ", "ATT_DONE", "ATT_COMB"]
EV = {e: i for i, e in enumerate(EVENTS)}
HOPS = [("q/k/v -> attention", "QKV_PUB", "ATT_IN"), ("partials -> merge", "ATT_PUB", "MERGE_PUB"),
        ("merged o -> all", "MERGE_PUB", "O_GOT"), ("xa (after O)", "XA_PUB", "XA_GOT"),
        ("h (after gate/up)", "H_PUB", "H_GOT"), ("xf (after down)", "XF_PUB", "XF_GOT")]
TRACE_WORDS, TRACE_HOP, WAVES = 64, 32, 8
TICK_NS = 10.0


def build():
    from hbm_bandwidth_bound_amd import build as b
    b.build(extra=["-DKIE_TRACE_HOPS"], out=HOPS_LIB)
    print("built", HOPS_LIB)


def collect(workload: str, steps: int):
    import torch
    from hbm_bandwidth_bound_amd import kie, synth
    if not os.path.exists(HOPS_LIB):
        raise RuntimeError(f"{HOPS_LIB} is missing: run the build step first")
    kie._lib = None
    kie.LIB_PATH = HOPS_LIB
    lib = kie.load()
    lib.kie_trace_offset.argtypes = [C.POINTER(kie.kie_config)]
    lib.kie_trace_offset.restype = C.c_int64
    wl = synth.WORKLOADS[workload]
    m = wl.model
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    w = synth.make_weights_torch(m, wl.weight_seed, device=dev)
    P = wl.prompt_len
    eng = kie.Engine(m, w, P + steps)
    prompt = torch.tensor(synth.prompt_ids(P, m.vocab_size, wl.prompt_seed), dtype=torch.int32, device=dev)
    first = eng.prefill(prompt)
    out = torch.empty(steps, dtype=torch.int32, device=dev)
    eng.generate(first, steps, out)
    eng.sync()
    off = lib.kie_trace_offset(C.byref(eng.cfg))
    nwg = lib.kie_num_workgroups()
    tr = eng.workspace[off:off + nwg * WAVES * TRACE_WORDS * 8].view(torch.int64).cpu().numpy()
    tr = tr.reshape(nwg, WAVES, TRACE_WORDS)
    eng.close()
    del eng, w
    torch.cuda.synchronize()
    hop = tr[:, 0, TRACE_HOP:TRACE_HOP + len(EVENTS)].astype(np.float64)
    bat = tr[:, 1, TRACE_HOP:TRACE_WORDS].astype(np.float64)
    return hop, bat, nwg


def report(workload, hop, bat, nwg, cmd):
    stamped = hop > 0
    t0 = hop[:, EV["QKV_IN"]].min()
    hop = np.where(stamped, (hop - t0) * TICK_NS, np.nan)
    bat = np.where(bat > 0, (bat - t0) * TICK_NS, np.nan)
    grp = np.arange(nwg) % 8  # workgroups sharing a chiplet
    L = [f"# Decode hop timeline, {workload} ({nwg} workgroups)", "", f"Command: `{cmd}`", "",
         "One sampled step and layer; times in ns from the first workgroup entering the layer's QKV "
         "boundary; wave 0 of each workgroup. Workgroups without attention work leave the attention "
         "stamps empty.", "", "| event | min | median | max | spread |", "|---|---|---|---|---|"]
    for e in EVENTS:
        v = hop[:, EV[e]]
        v = v[~np.isnan(v)]
        if len(v):
            L.append(f"| {e} | {v.min():.0f} | {np.median(v):.0f} | {v.max():.0f} | {v.max() - v.min():.0f} |")
    L += ["", "## Exchanges", "",
          "Publication spread = skew between the first and the last workgroup publishing; gathered = from the "
          "last publication to each workgroup holding every word (mean per group of workgroups sharing a "
          "chiplet, w mod 8).", "",
          "| exchange | publication spread | gathered: mean | min | max | per chiplet group 0..7 |",
          "|---|---|---|---|---|---|"]
    all_lat = []
    has_att = ~np.isnan(hop[:, EV["ATT_IN"]])
    for name, pub, got in HOPS:
        p = hop[:, EV[pub]]
        if pub == "ATT_PUB":  # only workgroups with attention work publish partials
            p = np.where(has_att, p, np.nan)
        g = hop[:, EV[got]]
        ok = ~np.isnan(g)
        last = np.nanmax(p)
        lat = g[ok] - last
        all_lat.append((name, lat))
        per = [np.nanmean(np.where(ok & (grp == x), g - last, np.nan)) for x in range(8)]
        L.append(f"| {name} | {np.nanmax(p) - np.nanmin(p):.0f} | {lat.mean():.0f} | {lat.min():.0f} | "
                 f"{lat.max():.0f} | " + ", ".join(f"{v:.0f}" for v in per) + " |")
    edges = [-1e9, 0, 500, 1000, 1500, 2000, 2500, 3000, 4000, 5000, 1e9]
    L += ["", "Histogram of the gathered latency over workgroups (ns after the last publication; negative: the "
          "workgroup held the words before the last publisher's stamp):", "",
          "| exchange | " + " | ".join(f"<{e:.0f}" if k == 0 else f"{edges[k]:.0f}-{edges[k + 1]:.0f}"
                                       if edges[k + 1] < 1e8 else f">{edges[k]:.0f}" for k, e in enumerate(edges[1:])) + " |",
          "|---" * len(edges) + "|"]
    for name, lat in all_lat:
        h, _ = np.histogram(lat, bins=edges)
        L.append(f"| {name} | " + " | ".join(str(x) for x in h) + " |")

    def d(a, b):
        v = hop[:, EV[b]] - hop[:, EV[a]]
        v = v[~np.isnan(v)]
        return f"median {np.median(v):.0f}, min {v.min():.0f}, max {v.max():.0f}" if len(v) else "n/a"
    L += ["", "## Stages and phases (per workgroup)", "",
          f"* O GEMV (O_GOT -> O_IN): {d('O_GOT', 'O_IN')}",
          f"* gate/up GEMV (XA_GOT -> GU_IN): {d('XA_GOT', 'GU_IN')}",
          f"* down GEMV (H_GOT -> DN_IN): {d('H_GOT', 'DN_IN')}",
          f"* attention: poll -> all waves hold the inputs: {d('ATT_IN', 'ATT_ALLQ')}; scores and values: "
          f"{d('ATT_ALLQ', 'ATT_DONE')}; combine over waves and publish: {d('ATT_DONE', 'ATT_COMB')}",
          f"* layer (QKV_IN -> NORM_DONE): {d('QKV_IN', 'NORM_DONE')}", "",
          "## Wave 0's weight batches of the layer", "",
          "Time from the workgroup's QKV_IN (median over workgroups): taken = handed to the reduction, "
          "reduced = its dot products done.", "", "| batch | taken | reduced |", "|---|---|---|"]
    base = hop[:, EV["QKV_IN"]]
    for i in range(16):
        tk, rd = bat[:, 2 * i], bat[:, 2 * i + 1]
        if np.all(np.isnan(tk)):
            break
        L.append(f"| {i} | {np.nanmedian(tk - base):.0f} | {np.nanmedian(rd - base):.0f} |")
    return "\n".join(L) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("cmd", choices=["build", "run"])
    ap.add_argument("--workload", default="1.6b-1k")
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    if args.cmd == "build":
        build()
        return
    hop, bat, nwg = collect(args.workload, args.steps)
    text = report(args.workload, hop, bat, nwg, "python3 -m hbm_bandwidth_bound_amd.hop_profile " + " ".join(sys.argv[1:]))
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
