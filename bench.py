#!/usr/bin/env python3
"""Batch-1 decode benchmark: tokens/s and achieved HBM bandwidth of the decode monokernel.

Default workload: the ~1.6B dense decoder (24 layers, d 2048, 16/8 heads, hd 128, FFN 8192,
vocab 32768, bf16 weights and KV) with a 1024-token random-id prompt; a "step" is one decoded
token (one pass of the whole decode path). The W warm-up steps run as one kie_generate launch
and the K timed steps as another, both starting at position 1024 (the position is rewound after
the warm-up), so with W = K (the default) every decode-kernel dispatch of a run has the same
length and a profiler's per-dispatch average is the timed launch's duration.

Prints one JSON line. `roofline.achieved` is the algorithmic bytes of the timed launch divided
by that launch's duration (HIP events on the launch stream); `cpu_baseline` times the CPU oracle
on a bounded sample of the same workload. Other workloads: `--workload 1.6b-32k`, `8b-2k`, and
`moe-1k` (the 128-expert model with 8 experts routed per token; its CPU baseline is the oracle
on 2- and 4-layer cuts of the model, scaled).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
HEADLINE_METRIC = "batch-1 decode tok/s, 1.6B bf16 @1k ctx; achieved HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=None, help="warm-up steps (default: the same as --steps)")
    ap.add_argument("--workload", default="1.6b-1k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--repeats", type=int, default=5,
                    help="greedy launches of the same K steps after the timed one, reported as median and "
                         "stdev; 0 = skip")
    ap.add_argument("--single-step-launches", type=int, default=0,
                    help="also time this many one-token launches (launch-overhead comparison); 0 = skip")
    return ap.parse_args()


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*([a-z_]+)\s*=\s*(\S+)", line)
            if m:
                kv[m.group(1)] = m.group(2)
    from hbm_bandwidth_bound_amd.build import source_hash
    if kv.get("source_sha") != source_hash():
        return None
    try:
        return {"bytes_per_step": float(kv["hbm_bytes_per_step"]), "steps_per_launch": int(kv["steps_per_launch"])}
    except (KeyError, ValueError):
        return None


def _oracle_steps(model, w_np, prompt_len: int, target_s: float, max_steps: int = 64):
    """(steps, seconds) of oracle decode steps at positions prompt_len.. The oracle's KV cache is
    filled with seeded synthetic bf16 rows for positions < prompt_len (the cost of a step does not
    depend on their values)."""
    import oracle
    from hbm_bandwidth_bound_amd import synth
    om = oracle.OracleModel(model, w_np, prompt_len + max_steps)
    k, v = om.kv_view()
    rows = synth._weights_bits_np((model.n_layers * model.n_kv_heads * prompt_len, model.head_dim), 7, 999)
    rows = rows.reshape(model.n_layers, model.n_kv_heads, prompt_len, model.head_dim)
    k[:, :, :prompt_len] = rows
    v[:, :, :prompt_len] = rows[:, :, ::-1]
    tok = int(synth.prompt_ids(1, model.vocab_size, 1)[0])
    n = 0
    t0 = time.perf_counter()
    while True:
        logits = om.step(tok, prompt_len + n)
        tok = oracle.argmax(logits)
        n += 1
        el = time.perf_counter() - t0
        if el >= target_s or n >= max_steps:
            return n, el


def _oracle_rate(model, weights_dev, prompt_len: int, target_s: float, threads: int, w_np=None):
    """(tok/s, description) of the oracle at `threads` threads on the same model and context. A
    model too large to copy to the host whole (the mixture-of-experts one) is timed on two cuts of
    itself, its first 2 and first 4 layers with the real embedding and LM head; the per-layer time
    (their difference over 2 layers) then scales the 4-layer time to the full depth."""
    import oracle
    from hbm_bandwidth_bound_amd import synth
    oracle.set_threads(threads)
    if not model.n_experts:
        n, el = _oracle_steps(model, w_np, prompt_len, target_s)
        return n / el, (f"{n} oracle decode steps of the {model.name} model at positions {prompt_len}.."
                        f"{prompt_len + n - 1} (KV rows < {prompt_len} seeded synthetic), {el:.1f} s")
    cut = {k: (v[:4] if isinstance(v, list) else v) for k, v in weights_dev.items()}
    w4 = synth.weights_torch_to_np(cut)
    w2 = {k: (v[:2] if isinstance(v, list) else v) for k, v in w4.items()}
    n2, e2 = _oracle_steps(model.scaled(n_layers=2), w2, prompt_len, target_s / 2, 16)
    n4, e4 = _oracle_steps(model.scaled(n_layers=4), w4, prompt_len, target_s / 2, 16)
    t2, t4 = e2 / n2, e4 / n4
    per_layer = max(t4 - t2, 0.0) / 2
    t_full = t4 + (model.n_layers - 4) * per_layer
    return 1.0 / t_full, (f"oracle decode steps at positions {prompt_len}.. of the {model.name} model cut to its "
                          f"first 2 layers ({n2} steps, {t2:.3f} s/step) and 4 layers ({n4} steps, {t4:.3f} "
                          f"s/step), real embedding and LM head; per-token time = t4 + {model.n_layers - 4} x "
                          f"(t4 - t2) / 2 = {t_full:.2f} s")


def cpu_baseline(model, weights_dev, prompt_len: int, target_s: float):
    """The oracle on the machine's host cores: one core (the reported value), then rows split over up
    to 16 threads (same arithmetic, bitwise the same results), each for about half the time."""
    import oracle
    from hbm_bandwidth_bound_amd import synth
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    threads = max(1, min(16, ncores))
    oracle.build(force=False)
    w_np = None if model.n_experts else synth.weights_torch_to_np(weights_dev)
    v1, d1 = _oracle_rate(model, weights_dev, prompt_len, target_s / 2, 1, w_np)
    vn, dn = _oracle_rate(model, weights_dev, prompt_len, target_s / 2, threads, w_np)
    oracle.set_threads(1)
    return {"value": v1, "unit": "tok/s", "cores": 1, "kind": "oracle", "sample": d1 + ", 1 thread",
            "box_cores": ncores,
            "threaded": {"value": vn, "unit": "tok/s", "threads": threads, "sample": dn + f", {threads} threads "
                         "(rows split over threads; each row's summation order unchanged)"}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this decode path has no multi-GPU "
              "mode", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from hbm_bandwidth_bound_amd import synth, traffic
    from hbm_bandwidth_bound_amd.build import source_hash
    from hbm_bandwidth_bound_amd.kie import Engine, stream_read

    wl = synth.WORKLOADS[args.workload]
    m = wl.model
    K = int(args.steps)
    W = K if args.warmup is None else int(args.warmup)
    P = wl.prompt_len
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] generating {m.name} weights on the GPU", file=sys.stderr, flush=True)
    wdev = synth.make_weights_torch(m, wl.weight_seed, device=dev)
    torch.cuda.synchronize()
    eng = Engine(m, wdev, P + max(K, W))
    prompt = torch.tensor(synth.prompt_ids(P, m.vocab_size, wl.prompt_seed), dtype=torch.int32, device=dev)

    # prompt pass (untimed for the metric; its time is reported as TTFT). The first call in the
    # process also pays one-time kernel loading; the second, over the same prompt from position
    # 0 (it rewrites the same cache rows), is the time a warm engine takes.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ttft = []
    for rep in range(2):
        print(f"[bench] prompt pass of {P} tokens ({'first call' if rep == 0 else 'warm'})", file=sys.stderr, flush=True)
        eng.reset()
        e0.record(stream)
        first = eng.prefill(prompt)
        e1.record(stream)
        eng.sync()
        ttft.append(e0.elapsed_time(e1))
    ttft_ms = ttft[1]
    # the prompt pass's matrix products: 2 x (tokens - 1) x the layer weights a position uses (the
    # routed experts' only, with experts; the last position runs through the decode kernel), plus
    # the causal attention products. They run as matrix-core GEMMs (8-bit codes widened to bf16
    # operands as they are read; each expert's positions as its own products).
    mm = traffic.matrix_weights(m) - m.vocab_size * m.d_model
    attn = 4 * m.n_layers * m.n_heads * m.head_dim * (P - 1) * P // 2
    prefill_flops = 2 * (P - 1) * mm + attn
    prompt_pass = {"flops": prefill_flops, "tflops": round(prefill_flops / (ttft_ms * 1e-3) / 1e12, 1),
                   "frac_of_bf16_mfma_peak": round(prefill_flops / (ttft_ms * 1e-3) / 2.5e15, 4)}

    out = torch.empty(max(K, W), dtype=torch.int32, device=dev)
    if W > 0:
        print(f"[bench] warm-up {W} tokens", file=sys.stderr, flush=True)
        eng.generate(first, W, out)
        eng.sync()
        eng.set_position(P)
    print(f"[bench] timed: {K} tokens in one launch", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    eng.generate(first, K, out)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eng.sync()
    launch_ms = e0.elapsed_time(e1)
    wall_s = t1 - t0
    tok_s = K / wall_s
    algo_bytes = traffic.launch_bytes(m, P, K)
    achieved_gbps = algo_bytes / (launch_ms * 1e-3) / 1e9

    # the same K steps with top-k sampling (k 50, T 0.8, seed 2): one more launch
    from hbm_bandwidth_bound_amd.kie import sampling
    eng.set_position(P)
    torch.cuda.synchronize()
    e0.record(stream)
    eng.generate(first, K, out, smp=sampling(50, 0.8, 2))
    e1.record(stream)
    torch.cuda.synchronize()
    eng.sync()
    topk_tok_s = K / (e0.elapsed_time(e1) * 1e-3)

    # the timed launch repeated (same positions, same tokens): the spread of the rate on this machine
    reps = None
    if args.repeats > 0:
        rates = []
        for _ in range(args.repeats):
            eng.set_position(P)
            torch.cuda.synchronize()
            e0.record(stream)
            eng.generate(first, K, out)
            e1.record(stream)
            torch.cuda.synchronize()
            eng.sync()
            rates.append(K / (e0.elapsed_time(e1) * 1e-3))
        reps = {"launches": len(rates), "tok_s": [round(r, 2) for r in rates],
                "median": round(float(np.median(rates)), 2), "stdev": round(float(np.std(rates, ddof=1)), 2)
                if len(rates) > 1 else 0.0}

    # one-token launches (the per-launch overhead comparison)
    single = None
    if args.single_step_launches > 0:
        n1 = min(args.single_step_launches, K)
        eng.set_position(P)
        tok_in = first.clone()
        o = torch.empty(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n1):
            eng.decode_step(tok_in, o)
            tok_in, o = o, tok_in
        e1.record(stream)
        torch.cuda.synchronize()
        eng.sync()
        single = {"tokens": n1, "tok_s": n1 / (e0.elapsed_time(e1) * 1e-3)}

    # streaming-read ceiling of this GPU (plain kernel, 4 GiB)
    nb = 4 << 30
    buf = torch.empty(nb, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream_read(buf, nb, sink, stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(3):
        stream_read(buf, nb, sink, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ceiling_gbps = 3 * nb / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf

    tr = read_traffic(args.workload)
    traffic_bytes = None
    if tr is not None:
        traffic_bytes = tr["bytes_per_step"] * K

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(m, wdev, P, args.cpu_seconds)

    metric = HEADLINE_METRIC if args.workload == "1.6b-1k" else \
        f"batch-1 decode tok/s, {wl.name} {'fp8-e4m3 weights' if m.weight_format else 'bf16'}; achieved HBM GB/s vs peak"
    res = {
        "metric": metric,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall_s * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 weights, f32 activations" if m.weight_format else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "prompt_len": P, "decode_positions": [P, P + K - 1],
                   "sampling": "greedy",
                   "weights": ("e4m3fn codes of the seeded bf16 values x 128, one fp32 scale per matrix"
                               if m.weight_format else "bf16, counter-based N(0,0.02) approx., seed 0"),
                   "experts": (f"{m.n_experts_active} of {m.n_experts} routed per token, width {m.expert_ffn_dim}"
                               if m.n_experts else None),
                   "kv_cache": "bf16", "accumulate": "f32", "launches_per_timed_region": 1},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic_bytes},
        "cpu_baseline": cpu,
        "extra": {"kernel_ms": round(launch_ms, 3), "algorithmic_bytes": algo_bytes,
                  "bytes_per_token": algo_bytes / K, "stream_read_ceiling_GBps": round(ceiling_gbps, 1),
                  "frac_of_stream_ceiling": round(achieved_gbps / ceiling_gbps, 4),
                  "ttft_ms_prompt_pass": round(ttft_ms, 2), "ttft_ms_first_call": round(ttft[0], 2),
                  "prompt_pass": prompt_pass,
                  "one_token_launches": single,
                  "repeat_launches": reps,
                  "topk50_T0.8_tok_s": round(topk_tok_s, 2),
                  "source_sha": source_hash()},
    }
    print(json.dumps(res), flush=True)
    # explicit teardown before the interpreter exits: the context, every device tensor, then the
    # stream, so that nothing of the GPU runtime is released by exit handlers
    eng.close()
    del eng, wdev, prompt, out, first, sink
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
