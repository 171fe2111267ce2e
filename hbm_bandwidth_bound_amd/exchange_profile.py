#!/usr/bin/env python3
"""Exchange latency per chiplet (XCD) on the running GPU, from the probes of kie_measure.h.

The pages tie the decode step's synchronisation cost to the MI300X's chiplet topology (eight
compute dies on four I/O dies; extra latency across I/O dies) and report a grid barrier of ~600 ns
once each XCD polls a replica behind its own I/O die (aikraft.ru «3000 токенов в секунду…», §05).
This measures, with the decode kernel's own exchange words:

* ping-pong one-way latency for every pair of XCDs (8 x 8);
* the all-gather hop of the decode kernel (every workgroup publishes w words, gathers all), from
  one buffer and from one replica per XCD: the latency histogram over workgroups and rounds, and
  the per-XCD means;
* write-to-visible latency per location (4 KiB apart by default) and reader XCD, written from each
  XCD in turn: whether some locations are consistently nearer to some XCDs.

    python3 -m hbm_bandwidth_bound_amd.exchange_profile --out profiles/exchange_latency_mi355x.md
"""
import argparse
import ctypes as C
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICK_NS = 10.0  # s_memrealtime runs at 100 MHz
NX = 8


def _p(t):
    return C.c_void_p(t.data_ptr())


def _check(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def pingpong(lib, torch, iters):
    flags = torch.zeros(64, dtype=torch.int64, device="cuda")
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    m = np.zeros((NX, NX))
    for i in range(NX):
        for j in range(NX):
            flags.zero_()
            out.zero_()
            _check(lib.kie_probe_pingpong(i, NX + j, iters, _p(flags), _p(out), None), "ping-pong")
            torch.cuda.synchronize()
            ticks, xa, xb = (int(v) for v in out.cpu())
            if ticks == 0:
                raise RuntimeError(f"ping-pong {i} <-> {NX + j} gave up")
            if (xa, xb) != (i, j):
                print(f"note: workgroups {i} and {NX + j} ran on XCDs {xa} and {xb}")
            m[xa, xb] = ticks * TICK_NS / (2 * iters)
    return m


def allgather(lib, torch, nwg, wpw, reps, rounds):
    ex = torch.zeros(2 * reps * nwg * wpw, dtype=torch.int64, device="cuda")
    lat = torch.zeros(nwg * rounds, dtype=torch.int32, device="cuda")
    xcc = torch.zeros(nwg, dtype=torch.int32, device="cuda")
    fail = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib.kie_probe_allgather(wpw, rounds, reps, _p(ex), _p(lat), _p(xcc), _p(fail), None), "all-gather")
    torch.cuda.synchronize()
    if int(fail.item()):
        raise RuntimeError(f"all-gather wpw={wpw} reps={reps} gave up")
    lat = lat.cpu().numpy().astype(np.uint32).reshape(nwg, rounds).astype(np.float64) * TICK_NS
    return lat[:, rounds // 10:], xcc.cpu().numpy()  # the first tenth warms up


def page_latency(lib, torch, npages, page_words):
    buf = torch.zeros(npages * page_words, dtype=torch.int64, device="cuda")
    acks = torch.zeros(512, dtype=torch.int64, device="cuda")
    out = torch.zeros(npages * NX, dtype=torch.int32, device="cuda")
    fail = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = np.zeros((NX, npages, NX))
    wxcc = []
    for wx in range(NX):  # writer: workgroup wx
        buf.zero_()
        acks.zero_()
        fail.zero_()
        _check(lib.kie_probe_page_latency(npages, page_words, wx, _p(buf), _p(acks), _p(out), _p(fail), None),
               "page latency")
        torch.cuda.synchronize()
        if int(fail.item()):
            raise RuntimeError(f"page latency writer {wx} gave up")
        res[wx] = out.cpu().numpy().astype(np.uint32).reshape(npages, NX).astype(np.float64) * TICK_NS
        wxcc.append(int(acks[NX * 32].item()))
    return res, wxcc


def hist_lines(v, edges):
    h, _ = np.histogram(v, bins=edges)
    tot = max(1, len(v))
    out = []
    for k in range(len(h)):
        out.append(f"| {edges[k]:6.0f} - {edges[k + 1]:6.0f} | {h[k]:7d} | {100.0 * h[k] / tot:5.1f}% |")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--iters", type=int, default=2000)
    ap.add_argument("--rounds", type=int, default=2000)
    ap.add_argument("--pages", type=int, default=256)
    ap.add_argument("--page-words", type=int, default=512, help="words between probed locations (512 = 4 KiB)")
    args = ap.parse_args()

    import torch
    from hbm_bandwidth_bound_amd import kie
    lib = kie.load()
    torch.cuda.set_device(0)
    nwg = lib.kie_num_workgroups()
    name = torch.cuda.get_device_name(0)
    lines = [f"# Exchange latency per XCD ({name}, {nwg} compute units)", "",
             "Command: `python3 -m hbm_bandwidth_bound_amd.exchange_profile " + " ".join(sys.argv[1:]) + "`", ""]
    print(lines[0], flush=True)

    m = pingpong(lib, torch, args.iters)
    lines += ["## Ping-pong, one-way latency (ns): row = XCD of the first workgroup, column = XCD of the second",
              "", "| | " + " | ".join(f"XCD {j}" for j in range(NX)) + " |", "|---" * (NX + 1) + "|"]
    for i in range(NX):
        lines.append(f"| XCD {i} | " + " | ".join(f"{m[i, j]:.0f}" for j in range(NX)) + " |")
    same = np.mean(np.diag(m))
    other = (m.sum() - np.trace(m)) / (NX * NX - NX)
    lines += ["", f"Same XCD: {same:.0f} ns mean; different XCDs: {other:.0f} ns mean "
              f"(min {m.min():.0f}, max {m.max():.0f}).", ""]
    print(f"ping-pong: same XCD {same:.0f} ns, other XCDs {other:.0f} ns", flush=True)

    edges = [0, 500, 750, 1000, 1250, 1500, 1750, 2000, 2500, 3000, 4000, 6000, 1e9]
    summary = []
    for wpw, label in ((8, "2048 words: the residual-stream hops (d = 2048)"),
                       (32, "8192 words: the FFN hop (F = 8192)")):
        for reps in (1, NX):
            lat, xcc = allgather(lib, torch, nwg, wpw, reps, args.rounds)
            flat = lat.ravel()
            per_x = [lat[xcc % NX == x].mean() for x in range(NX)]
            q = np.percentile(flat, [50, 90, 99])
            tag = "one buffer" if reps == 1 else "one replica per XCD"
            summary.append((wpw, reps, q[0], q[1], q[2], flat.mean()))
            lines += [f"## All-gather hop, {label}; {tag}", "",
                      f"{lat.shape[0]} workgroups x {lat.shape[1]} rounds. Latency from a workgroup's "
                      "publication to its gather being complete (includes waiting for the last publisher).",
                      "", f"p50 {q[0]:.0f} ns, p90 {q[1]:.0f} ns, p99 {q[2]:.0f} ns, mean {flat.mean():.0f} ns; "
                      "per-XCD mean: " + ", ".join(f"{v:.0f}" for v in per_x) + " ns", "",
                      "| ns | count | share |", "|---|---|---|"] + hist_lines(flat, edges) + [""]
            print(f"all-gather wpw={wpw} reps={reps}: p50 {q[0]:.0f} p90 {q[1]:.0f} p99 {q[2]:.0f} ns", flush=True)

    pl, wxcc = page_latency(lib, torch, args.pages, args.page_words)
    # the reader on the writer's own XCD sees a write sooner wherever it lands: leave it out when
    # asking which XCD a location is nearest to
    masked = pl.copy()
    for wx in range(NX):
        masked[wx, :, wxcc[wx] % NX] = np.inf
    near = masked.argmin(axis=2)  # [writer][location]: nearest other reader XCD
    spread = pl.max(axis=2) - pl.min(axis=2)
    by_reader = pl.mean(axis=(0, 1))
    agree = np.mean([np.mean(near[a] == near[b]) for a in range(NX) for b in range(NX) if a != b])
    loc_mean = pl.mean(axis=(0, 2))  # per location, over writers and readers
    stride = args.page_words * 8
    lines += [f"## Write-to-visible latency per location ({stride} bytes apart)", "",
              f"{args.pages} locations, written from each XCD in turn, read by one workgroup per XCD. "
              "Mean by reader XCD (ns): " + ", ".join(f"{v:.0f}" for v in by_reader) + ".",
              f"Median spread over readers per location: {np.median(spread):.0f} ns. Agreement of the nearest "
              f"reader XCD per location between different writers: {100 * agree:.0f}% (12.5% = chance): "
              + ("locations have a consistent nearest XCD." if agree > 0.4 else
                 "no location is consistently nearer to one XCD at this granularity."), "",
              f"Per-location mean over all writer/reader pairs: {loc_mean.min():.0f} .. {loc_mean.max():.0f} ns "
              f"(standard deviation {loc_mean.std():.0f} ns).", "",
              "| writer (XCD) | mean ns by reader XCD 0..7 |", "|---|---|"]
    for wx in range(NX):
        lines.append(f"| {wx} ({wxcc[wx]}) | " + ", ".join(f"{v:.0f}" for v in pl[wx].mean(axis=0)) + " |")
    lines += ["", "## Against the pages", "",
              "The pages report a grid barrier of ~600 ns on the MI300X once every XCD polls a replica "
              "behind its own I/O die, and up to ~150 ns of extra latency across I/O dies. Here:",
              f"ping-pong one-way {same:.0f} ns within an XCD and {other:.0f} ns across; the all-gather hop "
              "p50 " + ", ".join(f"{s[2]:.0f} ns ({s[0] * nwg} words, {'replicated' if s[1] > 1 else 'one buffer'})"
                                   for s in summary) + "."]
    print(f"pages: nearest-XCD agreement {100 * agree:.0f}%, median spread {np.median(spread):.0f} ns", flush=True)
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        print(text)


if __name__ == "__main__":
    main()
