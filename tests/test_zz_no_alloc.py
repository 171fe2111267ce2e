"""kie_create_static (the workspace in the library's static per-GPU array) against kie_create
(caller's workspace), through the C ABI (needs an MI355X).

Two calls in a row, the second on a smaller configuration: each static context's prompt logits,
decode logits and tokens match those of a kie_create context of the same model within rel-L2
1e-3 (the static context's prompt runs through the decode program, the other's through the
matrix-core pass, so the two differ by float32 rounding only). The earlier static context is
refused once a later one has taken over the array.
"""
import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests.gpu_util import rel_l2, say, to_device

pytestmark = pytest.mark.gpu


def _run(torch, eng, prompt, N, V):
    last = torch.empty(V, dtype=torch.float32, device="cuda")
    first = eng.prefill(torch.tensor(prompt, dtype=torch.int32, device="cuda"), logits_out=last)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, V), dtype=torch.float32, device="cuda")
    eng.generate(first, N, out, logits, forced=None)
    eng.sync()
    return int(first.item()), last.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy()


def _compare(a, b, label):
    fa, la, ta, ga = a
    fb, lb, tb, gb = b
    e = rel_l2(lb, la)
    worst = max(rel_l2(gb[s], ga[s]) for s in range(len(ga)))
    say(f"  {label}: prompt logits rel-L2 {e:.3e}, decode worst {worst:.3e}")
    assert e <= 1e-3 and worst <= 1e-3
    # tokens agree wherever the reference's choice is clear
    for s in range(len(ga)):
        srt = np.sort(ga[s])
        if srt[-1] - srt[-2] > 0.05:
            assert tb[s] == ta[s], (label, s)


def test_static_workspace_matches_the_callers_workspace():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hbm_bandwidth_bound_amd.kie import Engine, KieError
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    wd = to_device(w)
    runs = [(96, synth.prompt_ids(40, cfg.vocab_size, 1), 24), (24, synth.prompt_ids(12, cfg.vocab_size, 2), 6)]
    prev = None
    for i, (max_seq, prompt, N) in enumerate(runs):
        say(f"[static workspace] call {i + 1}: max_seq {max_seq}, prompt {len(prompt)} + decode {N}")
        ref_eng = Engine(cfg, wd, max_seq)
        ref = _run(torch, ref_eng, prompt, N, cfg.vocab_size)
        ref_eng.close()
        eng = Engine(cfg, wd, max_seq, static_workspace=True)
        assert eng.workspace is None
        got = _run(torch, eng, prompt, N, cfg.vocab_size)
        _compare(ref, got, f"call {i + 1}")
        if prev is not None:  # the earlier static context no longer owns the array
            out = torch.empty(2, dtype=torch.int32, device="cuda")
            with pytest.raises(KieError) as ei:
                prev.generate(torch.tensor([1], dtype=torch.int32, device="cuda"), 2, out)
            assert ei.value.status == -5
            prev.close()
        prev = eng
    prev.close()
