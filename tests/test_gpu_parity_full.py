"""GPU path vs the CPU oracle and the float64 reference at full depth (needs an MI355X).

Bars (the same for every test here):
* Cuts of a full shape to two layers, where the oracle itself lies within 5e-4 of the float64
  reference: every compared logits vector and K/V cache within rel-L2 1e-3 of the oracle (flat).
* Full depth (24 layers at 1.6B, 32 at 8B): two correct float32 renditions drift apart by more
  than 1e-3 there, because bf16 rounding of K/V entries that lie within float32 noise of a
  rounding boundary goes either way and later layers amplify it. Each vector is therefore held to
  rel-L2(GPU, fp64) <= rel-L2(oracle, fp64) + 1e-3 against the float64 reference
  (tests/fp64_ref.py), which separates an arithmetic error (the GPU far from the exact value)
  from that amplified rounding noise. Greedy tokens must equal the oracle's argmax wherever its
  top-2 gap exceeds 0.05.
Every distance is printed.
"""
import os

import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests import fp64_ref
from tests.gpu_util import (check_against_fp64, check_steps, check_topk_steps, greedy_where_decided, rel_l2, say,
                            top2_gap)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _threads(oracle_lib):
    oracle_lib.set_threads(min(16, os.cpu_count() or 1))  # rows only: results do not change


def _gpu_prompt_and_decode(torch, cfg, wd, prompt, N, smp=None):
    """The benchmark's path: kie_prefill (matrix-core prompt pass + the last position through the
    decode program), then one kie_generate launch of N steps. Returns (first token, last prompt
    logits, tokens, logits, KV cache [L][2][nkv][P + N][hd] bf16 bits)."""
    from hbm_bandwidth_bound_amd.kie import Engine
    P = len(prompt)
    eng = Engine(cfg, wd, P + N)
    tokens = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
    last = torch.empty(cfg.vocab_size, dtype=torch.float32, device="cuda")
    first = eng.prefill(tokens, logits_out=last)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
    eng.generate(first, N, out, logits, smp=smp)
    eng.sync()
    kv = eng.kv_view()[:, :, :, :P + N].cpu().numpy().view(np.uint16)
    res = int(first.item()), last.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy(), kv
    eng.close()
    return res


def test_headline_chain_1_6b_1k(torch_cuda, oracle_lib):
    """The benchmark's workload chain on the full 24-layer 1.6B model: a 1024-token prompt through
    the matrix-core prompt pass, then 4 decode steps in one launch at positions 1024..1027 with
    the production attention split. The GPU's KV cache is handed to the oracle and to the float64
    reference (the KV handoff), which then compute the last prompt position (over rows < 1023)
    and the 4 decode steps (over rows < 1024, teacher-forced on the GPU's tokens)."""
    torch = torch_cuda
    cfg = synth.M1_6B
    P, N = 1024, 4
    say(f"[1.6b headline chain] prompt {P} (matrix cores) + decode {N}")
    wd = synth.make_weights_torch(cfg, 0, "cuda")
    prompt = synth.prompt_ids(P, cfg.vocab_size, 1)
    first, last, toks, logits, kv = _gpu_prompt_and_decode(torch, cfg, wd, prompt, N)
    w = synth.weights_torch_to_np(wd)
    del wd
    torch.cuda.empty_cache()
    _threads(oracle_lib)
    kg, vg = kv[:, 0], kv[:, 1]
    decode_in = [first] + [int(t) for t in toks[:-1]]
    # the oracle over the GPU's cache
    om = oracle_lib.OracleModel(cfg, w, P + N)
    ko, vo = om.kv_view()
    ko[:, :, :P - 1] = kg[:, :, :P - 1]
    vo[:, :, :P - 1] = vg[:, :, :P - 1]
    ora_last = om.step(int(prompt[-1]), P - 1)
    ko[:, :, :P] = kg[:, :, :P]
    vo[:, :, :P] = vg[:, :, :P]
    ora = om.run(decode_in, start_pos=P)
    # the float64 reference over the same cache
    say("  float64 reference ...")
    ref = fp64_ref.Fp64Decoder(cfg, w)
    ref_last = ref.run([int(prompt[-1])], P - 1, kg, vg)[0][0]
    ref_dec, kr, vr = ref.run(decode_in, P, kg, vg)
    check_against_fp64(last, ora_last, ref_last, "prompt position 1023")
    if top2_gap(ora_last) > 0.05:
        assert first == int(np.argmax(ora_last))
    for s in range(N):
        check_against_fp64(logits[s], ora[s], ref_dec[s], f"decode position {P + s}")
    n = greedy_where_decided(toks, ora, label="1.6b headline")
    say(f"  greedy checked on {n}/{N} decode steps")
    # the K/V rows the decode steps appended
    f = synth.bf16_bits_to_f32
    check_against_fp64(f(kg[:, :, P:]), f(ko[:, :, P:P + N]), f(kr), "appended K rows")
    check_against_fp64(f(vg[:, :, P:]), f(vo[:, :, P:P + N]), f(vr), "appended V rows")


def test_1_6b_two_layer_cut_prompt_1024(torch_cuda, oracle_lib):
    """The 1.6B shape cut to two layers with the same 1024-token prompt pass: every prompt K/V row
    the matrix cores wrote, the last prompt logits and 4 decode steps are held to 1e-3 flat against
    the oracle, which computes the whole prompt itself; at this depth the oracle lies within 5e-4
    of the float64 reference."""
    torch = torch_cuda
    cfg = synth.M1_6B.scaled(name="1.6b-2l", n_layers=2)
    P, N = 1024, 4
    say(f"[1.6b cut to 2 layers] prompt {P} + decode {N}")
    wd = synth.make_weights_torch(cfg, 0, "cuda")
    prompt = synth.prompt_ids(P, cfg.vocab_size, 1)
    first, last, toks, logits, kv = _gpu_prompt_and_decode(torch, cfg, wd, prompt, N)
    w = synth.weights_torch_to_np(wd)
    del wd
    torch.cuda.empty_cache()
    _threads(oracle_lib)
    om = oracle_lib.OracleModel(cfg, w, P + N)
    ora_prompt = om.run(prompt)
    decode_in = [first] + [int(t) for t in toks[:-1]]
    ora = om.run(decode_in, start_pos=P)
    ko, vo = om.kv_view()
    f = synth.bf16_bits_to_f32
    for l in range(cfg.n_layers):
        ek = rel_l2(f(kv[l, 0, :, :P]), f(ko[l, :, :P]))
        ev = rel_l2(f(kv[l, 1, :, :P]), f(vo[l, :, :P]))
        say(f"  layer {l} prompt K rows rel-L2 {ek:.3e}, V rows {ev:.3e}")
        assert ek <= 1e-3 and ev <= 1e-3
    e = rel_l2(last, ora_prompt[-1])
    say(f"  last prompt logits rel-L2 {e:.3e}")
    assert e <= 1e-3
    if top2_gap(ora_prompt[-1]) > 0.05:
        assert first == int(np.argmax(ora_prompt[-1]))
    worst, checked = check_steps(logits, ora, toks, tol=1e-3, label="1.6b-2l")
    say(f"  decode worst rel-L2 {worst:.3e}, greedy checked on {checked}/{N} steps")
    # the premise of the flat bar: the oracle is within 5e-4 of the float64 reference here
    ref = fp64_ref.Fp64Decoder(cfg, w)
    ref_all = ref.run(list(prompt) + decode_in)[0]
    d = max(rel_l2(ora_prompt[-1], ref_all[P - 1]), max(rel_l2(ora[s], ref_all[P + s]) for s in range(N)))
    say(f"  oracle-fp64 at this depth {d:.3e}")
    assert d <= 5e-4


def test_long_context_over_synthetic_kv(torch_cuda, oracle_lib):
    """1.6B at the long-context length (32768 cached positions): the GPU, the oracle and the
    float64 reference start from the same seeded synthetic K/V rows (the oracle cannot prefill 32k
    tokens), then decode 3 steps. Every attention split, chunk length and merge runs at its
    production size."""
    torch = torch_cuda
    from hbm_bandwidth_bound_amd.kie import Engine
    cfg = synth.M1_6B
    n, N = 32768, 3
    say(f"[1.6b] {n} synthetic cached positions + decode {N}")
    wd = synth.make_weights_torch(cfg, 0, "cuda")
    eng = Engine(cfg, wd, n + N)
    kd, vd = synth.synthetic_kv_torch(cfg, n, seed=7, device="cuda")
    kvv = eng.kv_view()
    kvv[:, 0, :, :n] = kd
    kvv[:, 1, :, :n] = vd
    eng.set_position(n)
    tok0 = int(synth.prompt_ids(1, cfg.vocab_size, 5)[0])
    first = torch.tensor([tok0], dtype=torch.int32, device="cuda")
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
    eng.generate(first, N, out, logits)
    eng.sync()
    toks, logits = out.cpu().numpy(), logits.cpu().numpy()
    kg_new = eng.kv_view()[:, :, :, n:n + N].cpu().numpy().view(np.uint16)
    kn, vn = kd.cpu().numpy().view(np.uint16), vd.cpu().numpy().view(np.uint16)
    eng.close()
    w = synth.weights_torch_to_np(wd)
    del wd, kd, vd, kvv
    torch.cuda.empty_cache()
    _threads(oracle_lib)
    run_in = [tok0] + [int(t) for t in toks[:-1]]
    om = oracle_lib.OracleModel(cfg, w, n + N)
    ko, vo = om.kv_view()
    ko[:, :, :n] = kn
    vo[:, :, :n] = vn
    ora = om.run(run_in, start_pos=n)
    say("  float64 reference ...")
    ref, kr, vr = fp64_ref.Fp64Decoder(cfg, w).run(run_in, n, kn, vn)
    for s in range(N):
        check_against_fp64(logits[s], ora[s], ref[s], f"decode position {n + s}")
    say(f"  greedy checked on {greedy_where_decided(toks, ora, label='32k')}/{N} steps")
    f = synth.bf16_bits_to_f32
    check_against_fp64(f(kg_new[:, 0]), f(ko[:, :, n:n + N]), f(kr), "appended K rows")
    check_against_fp64(f(kg_new[:, 1]), f(vo[:, :, n:n + N]), f(vr), "appended V rows")


def test_8b_shape_prefill_then_decode(torch_cuda, oracle_lib):
    """The ~8B shape (32 layers, d 4096, 32/8 heads, F 14336, vocab 128256: 4 query heads per KV
    head, 128256 LM rows) on a short context, each side computing its own prompt; then the same
    shape cut to two layers against the oracle at 1e-3 flat."""
    torch = torch_cuda
    cfg = synth.M8B
    P, N = 6, 3
    say(f"[8b] prefill {P} + decode {N}")
    wd = synth.make_weights_torch(cfg, 0, "cuda")
    prompt = synth.prompt_ids(P, cfg.vocab_size, 4)
    first, last, toks, logits, kv = _gpu_prompt_and_decode(torch, cfg, wd, prompt, N)
    w = synth.weights_torch_to_np(wd)
    del wd
    torch.cuda.empty_cache()
    _threads(oracle_lib)
    decode_in = [first] + [int(t) for t in toks[:-1]]
    om = oracle_lib.OracleModel(cfg, w, P + N)
    ora_prompt = om.run(prompt)
    ora = om.run(decode_in, start_pos=P)
    say("  float64 reference ...")
    ref = fp64_ref.Fp64Decoder(cfg, w).run(list(prompt) + decode_in)[0]
    check_against_fp64(last, ora_prompt[-1], ref[P - 1], f"prompt position {P - 1}")
    for s in range(N):
        check_against_fp64(logits[s], ora[s], ref[P + s], f"decode position {P + s}")
    say(f"  greedy checked on {greedy_where_decided(toks, ora, label='8b')}/{N} steps")
    del ref, om, ora_prompt, ora
    # two layers of the same shape (tensors of layers 0 and 1 are the full model's), flat bar
    cfg2 = cfg.scaled(name="8b-2l", n_layers=2)
    w2 = {k: (v[:2] if isinstance(v, list) else v) for k, v in w.items()}
    from tests.gpu_util import to_device
    first, last, toks, logits, kv = _gpu_prompt_and_decode(torch, cfg2, to_device(w2), prompt, N)
    om = oracle_lib.OracleModel(cfg2, w2, P + N)
    ora_prompt = om.run(prompt)
    ora = om.run([first] + [int(t) for t in toks[:-1]], start_pos=P)
    e = rel_l2(last, ora_prompt[-1])
    say(f"  8b-2l last prompt logits rel-L2 {e:.3e}")
    assert e <= 1e-3
    worst, checked = check_steps(logits, ora, toks, tol=1e-3, label="8b-2l")
    say(f"  8b-2l decode worst rel-L2 {worst:.3e}, greedy checked on {checked}/{N} steps")


def test_full_shape_topk_sampling(torch_cuda, oracle_lib):
    """Top-k on the full 1.6B model over a short prompt, k 50 at T 0.8 (the served setting) and
    k 4 at T 1: the GPU's draws equal the oracle sampler's on the GPU's own logits; the candidate
    sets and probabilities follow the oracle's logits within the softmax bound of their distance
    wherever the k-th/(k+1)-th gap exceeds twice that distance. At 24 layers the gaps around the
    50th logit are narrower than the distance, so k 50 is held at the sampler level only; the gaps
    between the few largest logits are wider, and the k 4 run checks the sets (and the tokens, where
    the draw is clear of the CDF boundaries) against the oracle at this depth."""
    torch = torch_cuda
    from hbm_bandwidth_bound_amd.kie import sampling
    cfg = synth.M1_6B
    P, N = 12, 4
    say(f"[1.6b top-k] prefill {P} + decode {N}, k 50 and k 4")
    wd = synth.make_weights_torch(cfg, 0, "cuda")
    prompt = synth.prompt_ids(P, cfg.vocab_size, 3)
    first, last, toks, logits, kv = _gpu_prompt_and_decode(torch, cfg, wd, prompt, N, smp=sampling(50, 0.8, 2))
    first4, _, toks4, logits4, _ = _gpu_prompt_and_decode(torch, cfg, wd, prompt, N, smp=sampling(4, 1.0, 5))
    assert first4 == first  # the prompt pass's token is the greedy one either way
    w = synth.weights_torch_to_np(wd)
    del wd
    torch.cuda.empty_cache()
    _threads(oracle_lib)
    om = oracle_lib.OracleModel(cfg, w, P + N)
    om.run(prompt)
    ora = om.run([first] + [int(t) for t in toks[:-1]], start_pos=P)
    nt, ns = check_topk_steps(logits, ora, toks, 50, 0.8, 2, P, p_tol="auto", label="1.6b top-k")
    say(f"  top-k 50: sets checked on {ns}/{N} steps, tokens on {nt}/{N}")
    # the oracle's cache rows < P stay; positions P.. are rewritten along the k 4 run's tokens
    ora4 = om.run([first] + [int(t) for t in toks4[:-1]], start_pos=P)
    nt4, ns4 = check_topk_steps(logits4, ora4, toks4, 4, 1.0, 5, P, p_tol="auto", label="1.6b top-4")
    say(f"  top-k 4: sets checked on {ns4}/{N} steps, tokens on {nt4}/{N}")
    assert ns4 >= 1, "no step of the k 4 run had a 4th/5th logit gap above twice the GPU-oracle distance"
