"""Failure handling of the decode launches, forced from the host (needs an MI355X).

Every kernel still ends normally: a tiny limit on the kernels' own bounded waits (with workgroups
idling pseudo-random times before each boundary) makes waits give up, and a host-written abort
word makes every workgroup stop at the end of its step. kie_sync reports the error, the context
refuses work until kie_reset, and after kie_reset it decodes correctly again.
"""
import time

import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests.gpu_util import check_steps, rel_l2, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def tiny(torch_cuda):
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    return cfg, w, to_device(w)


def _decode_matches_oracle(torch, eng, cfg, w, oracle_lib, P=16, N=8):
    """A fresh prompt and N decode steps on the context, against the oracle at 1e-3."""
    prompt = synth.prompt_ids(P, cfg.vocab_size, 9)
    last = torch.empty(cfg.vocab_size, dtype=torch.float32, device="cuda")
    first = eng.prefill(torch.tensor(prompt, dtype=torch.int32, device="cuda"), logits_out=last)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
    eng.generate(first, N, out, logits)
    eng.sync()
    om = oracle_lib.OracleModel(cfg, w, P + N)
    ref_prompt = om.run(prompt)
    assert rel_l2(last.cpu().numpy(), ref_prompt[-1]) <= 1e-3
    toks = out.cpu().numpy()
    ref = om.run([int(first.item())] + [int(t) for t in toks[:-1]], start_pos=P)
    check_steps(logits.cpu().numpy(), ref, toks, label="after recovery")


def test_wait_timeout_is_reported_and_reset_recovers(torch_cuda, tiny, oracle_lib):
    from hbm_bandwidth_bound_amd.kie import Engine, KieError
    torch = torch_cuda
    cfg, w, wd = tiny
    eng = Engine(cfg, wd, 256)
    say("[failure] 1 us wait limit with workgroups idling up to 63 x 3.4 us before each boundary")
    eng.set_skew(64)
    eng.set_wait_timeout(1)
    first = torch.tensor([5], dtype=torch.int32, device="cuda")
    out = torch.empty(32, dtype=torch.int32, device="cuda")
    eng.generate(first, 32, out)
    with pytest.raises(KieError) as ei:
        eng.sync()
    assert ei.value.status == -6, ei.value  # KIE_ERR_TIMEOUT
    with pytest.raises(KieError) as ei:  # the context refuses work until it is reset
        eng.generate(first, 4, out)
    assert ei.value.status == -5  # KIE_ERR_STATE
    eng.set_skew(0)
    eng.set_wait_timeout(0)
    eng.reset()
    _decode_matches_oracle(torch, eng, cfg, w, oracle_lib)
    eng.close()


def test_host_abort_word_stops_a_running_launch(torch_cuda, tiny, oracle_lib):
    from hbm_bandwidth_bound_amd.kie import Engine, KieError
    torch = torch_cuda
    cfg, w, wd = tiny
    n = 3000
    eng = Engine(cfg, wd, n + 64)
    word = torch.zeros(1, dtype=torch.int32).pin_memory()
    ring = torch.zeros(1 + 16, dtype=torch.int32).pin_memory()
    eng.set_abort_flag(word)
    eng.set_token_stream(ring)
    say(f"[failure] a {n}-step launch, aborted by the host while it runs")
    first = torch.tensor([7], dtype=torch.int32, device="cuda")
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    t0 = time.perf_counter()
    eng.generate(first, n, out)
    while int(ring[0]) < 10 and time.perf_counter() - t0 < 20:  # the launch is producing tokens
        time.sleep(0.0005)
    word[0] = 1
    with pytest.raises(KieError) as ei:
        eng.sync()
    assert ei.value.status == -7, ei.value  # KIE_ERR_ABORTED
    done = int(ring[0])
    say(f"  stopped after {done} of {n} tokens")
    assert 10 <= done < n
    word[0] = 0
    eng.set_token_stream(None)
    eng.reset()
    _decode_matches_oracle(torch, eng, cfg, w, oracle_lib)
    eng.set_abort_flag(None)
    eng.close()


def test_8bit_engine_created_on_a_side_stream(torch_cuda, oracle_lib):
    """kie_create clears the workspace and copies the 8-bit matrix scales on the context's own
    stream, in that order: a context created on a non-default stream gets its scales (with a
    zeroed scale table every logit would be 0)."""
    from hbm_bandwidth_bound_amd.kie import Engine
    torch = torch_cuda
    cfg = synth.TINY_FP8
    w = synth.make_weights_np(cfg, 0)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        wd = to_device(w)
        eng = Engine(cfg, wd, 16, stream=side)
        prompt = synth.prompt_ids(12, cfg.vocab_size, 1)
        last = torch.empty(cfg.vocab_size, dtype=torch.float32, device="cuda")
        eng.prefill(torch.tensor(prompt, dtype=torch.int32, device="cuda"), logits_out=last)
        eng.sync()
        got = last.cpu().numpy()
    ref = oracle_lib.OracleModel(cfg, w, 12).run(prompt)[-1]
    e = rel_l2(got, ref)
    say(f"[8-bit on a side stream] prompt logits rel-L2 {e:.3e}")
    assert np.abs(got).max() > 0 and e <= 1e-3
    eng.close()
