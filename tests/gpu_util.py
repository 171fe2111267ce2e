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
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    return {k: ([cv(x) for x in v] if isinstance(v, list) else cv(v)) for k, v in w_np.items()}


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
