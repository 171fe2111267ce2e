"""Helpers shared by the GPU tests (inputs, engine construction, comparisons)."""
from __future__ import annotations

import sys

import numpy as np

from hbm_bandwidth_bound_amd import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(w_np, device="cuda"):
    import torch

    def cv(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a if a.dtype == np.uint8 else a.view(np.int16)).to(device)

    # the 8-bit models' matrix scales stay a host array
    return {k: (v if k == "w_scale" else [cv(x) for x in v] if isinstance(v, list) else cv(v))
            for k, v in w_np.items()}


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def top2_gap(logits) -> float:
    s = np.sort(np.asarray(logits, dtype=np.float64))
    return float(s[-1] - s[-2])


def check_steps(gpu_logits, ref_logits, gpu_tokens, tol=1e-3, gap=0.05, label=""):
    """Per-step logits rel-L2 <= tol; greedy token == oracle argmax where the oracle's gap > `gap`.
    Returns (worst rel-L2, number of gap-qualified steps)."""
    worst = 0.0
    checked = 0
    for s in range(len(ref_logits)):
        e = rel_l2(gpu_logits[s], ref_logits[s])
        worst = max(worst, e)
        assert e <= tol, f"{label} step {s}: logits rel-L2 {e:.3e} > {tol}"
        if top2_gap(ref_logits[s]) > gap:
            checked += 1
            assert int(gpu_tokens[s]) == int(np.argmax(ref_logits[s])), f"{label} step {s}: greedy token differs"
    return worst, checked


def cdf_margin(p, u) -> float:
    """Distance of u from the nearest boundary of the running sums of p."""
    c = np.cumsum(np.asarray(p, dtype=np.float64))
    return float(np.min(np.abs(c - u)))


def kth_gap(z, k) -> float:
    """Gap between the k-th and (k+1)-th largest entries of z (inf if there is no (k+1)-th)."""
    s = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    return float(s[k - 1] - s[k]) if len(s) > k else float("inf")


def check_topk_steps(gpu_logits, ref_logits, gpu_tokens, k, temperature, seed, pos0, p_tol=1e-3, label=""):
    """Top-k draws of a run against the oracle's sampler.

    * Sampler: the oracle's top-k draw on the GPU's own logits gives the GPU's token at every
      step (both take the same fp32 z and fp64 probabilities; only a draw within 1e-9 of a CDF
      boundary may go either way).
    * Model: with dz = max |z_gpu - z_oracle|, wherever the oracle's k-th/(k+1)-th gap in z
      exceeds 2 dz both logits give the same top-k set, with probabilities within p_tol relative;
      where the two candidate orders agree and u is at least 1e-4 (and more than the summed
      probability differences) from every boundary of the oracle's CDF, the token is the oracle's.
    Returns (steps with the model-level token check, steps with the set check)."""
    import oracle
    tok_checked = set_checked = 0
    for s in range(len(gpu_tokens)):
        pos = pos0 + s
        tg, ig, pg, u = oracle.topk_sample(gpu_logits[s], k, temperature, seed, pos)
        if cdf_margin(pg, u) > 1e-9:
            assert int(gpu_tokens[s]) == tg, f"{label} step {s}: sampler draw {int(gpu_tokens[s])} != oracle sampler {tg}"
        if ref_logits is None:
            continue
        to, io, po, uo = oracle.topk_sample(ref_logits[s], k, temperature, seed, pos)
        assert u == uo
        t32 = np.float32(temperature)
        zg = np.asarray(gpu_logits[s], dtype=np.float32) / t32
        zr = np.asarray(ref_logits[s], dtype=np.float32) / t32
        dz = float(np.max(np.abs(zg.astype(np.float64) - zr)))
        if kth_gap(zr, k) > 2 * dz:
            set_checked += 1
            assert set(ig.tolist()) == set(io.tolist()), f"{label} step {s}: top-{k} sets differ"
            pm = dict(zip(ig.tolist(), pg.tolist()))
            rel = max(abs(pm[i] - q) / q for i, q in zip(io.tolist(), po.tolist()))
            # p_tol "auto": the softmax bound for logits that differ by at most dz (each log p_j
            # moves by at most 2 dz), for depths where the logits' own spread exceeds 1e-3
            bound = max(1e-3, float(np.expm1(2 * dz)) * 1.01) if p_tol == "auto" else p_tol
            assert rel <= bound, f"{label} step {s}: candidate probabilities differ by {rel:.2e} relative"
            if np.array_equal(ig, io) and cdf_margin(po, uo) >= max(1e-4, float(np.sum(np.abs(pg - po)))):
                tok_checked += 1
                assert int(gpu_tokens[s]) == to, f"{label} step {s}: token {int(gpu_tokens[s])} != oracle {to}"
    return tok_checked, set_checked


DEPTH_SLACK = 1e-3  # the one bar of every full-depth comparison: see check_against_fp64


def check_against_fp64(gpu, ora, ref64, label, slack=DEPTH_SLACK):
    """The rule for full-depth models, where the decoder amplifies float32 rounding (through bf16
    rounding flips of K/V entries) beyond 1e-3 between any two correct float32 renditions: the GPU
    must be no farther from the float64 reference than the oracle is, plus `slack`:
    rel-L2(GPU, fp64) <= rel-L2(oracle, fp64) + slack, per compared vector. Prints and returns
    (GPU-fp64, oracle-fp64, GPU-oracle)."""
    dg, do, dgo = rel_l2(gpu, ref64), rel_l2(ora, ref64), rel_l2(gpu, ora)
    say(f"  {label:<28} GPU-fp64 {dg:.3e}  oracle-fp64 {do:.3e}  GPU-oracle {dgo:.3e}")
    assert dg <= do + slack, f"{label}: GPU-fp64 {dg:.3e} > oracle-fp64 {do:.3e} + {slack}"
    return dg, do, dgo


def greedy_where_decided(gpu_tokens, ora_logits, gap=0.05, label=""):
    """Greedy tokens equal the oracle's argmax wherever the oracle's top-2 gap exceeds `gap`.
    Returns the number of steps checked."""
    n = 0
    for s in range(len(ora_logits)):
        if top2_gap(ora_logits[s]) > gap:
            n += 1
            assert int(gpu_tokens[s]) == int(np.argmax(ora_logits[s])), f"{label} step {s}: greedy token differs"
    return n
