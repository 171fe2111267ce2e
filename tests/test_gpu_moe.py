"""Mixture-of-experts decode on the GPU vs the CPU oracle, through the C ABI (needs an MI355X).

The router's choice is an integer decision taken from fp32 logits on both sides (the A largest,
ties to the lower index). The GPU's logits differ from the oracle's by rounding only (~1e-6
relative), so the comparison is meaningful where the oracle's gap between the A-th and (A+1)-th
router logit is well above that: every test first checks that this margin exceeds 1e-4 at every
(position, layer) it compares. Logits are then compared at every step (rel-L2 <= 1e-3), greedy
tokens wherever the oracle's top-2 gap exceeds 0.05, and the KV cache element-wise.
"""
import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests.gpu_util import check_steps, rel_l2, say, to_device, top2_gap

pytestmark = pytest.mark.gpu

ROUTE_MARGIN = 1e-4


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def run_gpu(torch, eng, prompt, n_steps, V):
    tokens = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
    last = torch.empty(V, dtype=torch.float32, device="cuda")
    first = eng.prefill(tokens, logits_out=last)
    out = torch.empty(n_steps, dtype=torch.int32, device="cuda")
    logits = torch.empty((n_steps, V), dtype=torch.float32, device="cuda")
    eng.generate(first, n_steps, out, logits)
    eng.sync()
    return int(first.item()), last.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy()


def route_margin(z, A):
    """Smallest gap between the A-th and (A+1)-th router logit over all (position, layer)."""
    s = np.sort(np.asarray(z, dtype=np.float64), axis=-1)[..., ::-1]
    return float(np.min(s[..., A - 1] - s[..., A]))


def compare(torch, oracle_lib, cfg, w, wd, P, N, seed, label):
    from hbm_bandwidth_bound_amd.kie import Engine
    say(f"[{label}] prompt {P} + decode {N}")
    eng = Engine(cfg, wd, P + N)
    prompt = synth.prompt_ids(P, cfg.vocab_size, seed)
    first, last, toks, logits = run_gpu(torch, eng, prompt, N, cfg.vocab_size)
    om = oracle_lib.OracleModel(cfg, w, P + N)
    z = om.record_routes(P + N)
    ref_prompt = om.run(prompt)
    ref = om.run([first] + [int(t) for t in toks[:-1]], start_pos=P)
    om.stop_recording()
    if cfg.n_experts_active < cfg.n_experts:  # (with every expert active there is no choice to flip)
        m = route_margin(z, cfg.n_experts_active)
        say(f"  smallest router margin {m:.2e}")
        assert m > ROUTE_MARGIN, f"{label}: a routing decision is within {ROUTE_MARGIN} of a tie; pick another seed"
    e = rel_l2(last, ref_prompt[-1])
    say(f"  prompt last-logits rel-L2 {e:.3e}")
    assert e <= 1e-3
    if top2_gap(ref_prompt[-1]) > 0.05:
        assert first == int(np.argmax(ref_prompt[-1]))
    worst, checked = check_steps(logits, ref, toks, label=label)
    say(f"  decode worst rel-L2 {worst:.3e}, greedy checked on {checked}/{N} steps")
    kg = eng.kv_view().cpu().numpy().view(np.uint16)
    ko, vo = om.kv_view()
    n = P + N
    ek = rel_l2(synth.bf16_bits_to_f32(kg[:, 0, :, :n]), synth.bf16_bits_to_f32(ko[:, :, :n]))
    ev = rel_l2(synth.bf16_bits_to_f32(kg[:, 1, :, :n]), synth.bf16_bits_to_f32(vo[:, :, :n]))
    say(f"  cache rel-L2 K {ek:.3e} V {ev:.3e}")
    assert ek <= 1e-3 and ev <= 1e-3
    eng.close()


@pytest.mark.parametrize("cfg", [synth.TINY_MOE, synth.SMALL_MOE], ids=lambda c: c.name)
def test_moe_prompt_then_decode(torch_cuda, oracle_lib, cfg):
    """16 experts of 1-tile rows with 4 active, and 32 experts of 3-tile rows with 8 active (each
    down-projection unit of 8 k-tiles then spans three experts)."""
    w = synth.make_weights_np(cfg, 0)
    compare(torch_cuda, oracle_lib, cfg, w, to_device(w), 40, 12, 1, cfg.name)


def test_moe_prompt_pass_two_chunks(torch_cuda, oracle_lib):
    """A 600-token prompt through the matrix-core prompt pass: two chunks of positions, each with
    its own expert token lists (every list holds the whole chunk here) and grouped products over
    them, then decode. Every position routes to all 8 experts: over a thousand routing decisions
    some would fall within rounding of a tie (the smallest margin of the 32-expert model over this
    prompt is 2e-6), while the ranking, the weights and the rank-order sum still run."""
    cfg = synth.ModelConfig("moe-all8", 2, 512, 8, 1, 128, 0, 4096, n_experts=8, n_experts_active=8,
                            expert_ffn_dim=256)
    oracle_lib.set_threads(16)
    try:
        w = synth.make_weights_np(cfg, 0)
        compare(torch_cuda, oracle_lib, cfg, w, to_device(w), 600, 3, 2, cfg.name + "-600")
    finally:
        oracle_lib.set_threads(1)


def test_moe_full_layer_shape(torch_cuda, oracle_lib):
    """The 128-expert model's layer shape (d 2048, 32/4 heads, 8 of 128 experts of width 768,
    vocabulary 151,936) with two layers: the launch geometry of the full model per layer."""
    cfg = synth.MOE_2L
    oracle_lib.set_threads(16)
    try:
        wd = synth.make_weights_torch(cfg, 0, device="cuda")
        w = synth.weights_torch_to_np(wd)
        compare(torch_cuda, oracle_lib, cfg, w, wd, 12, 4, 1, cfg.name)
    finally:
        oracle_lib.set_threads(1)


def test_moe_rejects_unsupported_shapes(torch_cuda):
    """Configurations the kernels do not handle are refused on the host, before any launch."""
    from hbm_bandwidth_bound_amd import kie
    lib = kie.load()
    ok = synth.TINY_MOE
    bad = [ok.scaled(n_experts=15), ok.scaled(n_experts_active=9, n_experts=16), ok.scaled(expert_ffn_dim=300),
           ok.scaled(ffn_dim=1024), ok.scaled(n_experts_active=17)]
    import ctypes as C
    assert lib.kie_packed_weight_bytes(C.byref(kie.make_config(ok, 64))) > 0
    for b in bad:
        assert lib.kie_packed_weight_bytes(C.byref(kie.make_config(b, 64))) == 0, b
    # a head grouping without a mixture-of-experts kernel instantiation
    g2 = ok.scaled(n_kv_heads=4)
    w = synth.make_weights_torch(g2, 0, device="cuda")
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(g2, w, 64)
    assert ei.value.status == -2


def test_moe_skewed_workgroups_give_bitwise_identical_results(torch_cuda):
    """Exchange protocol stress with the router hop: every workgroup idles a pseudo-random time
    before each boundary (kie_set_skew), so the workgroups reach the router gather, the expert
    choice and the routed stages in other orders; prompt, greedy and top-k decode must give
    bitwise the same tokens and logits as without."""
    from hbm_bandwidth_bound_amd.kie import Engine, sampling
    cfg = synth.SMALL_MOE
    w = synth.make_weights_np(cfg, 0)
    wd = to_device(w)
    P, N = 24, 8
    say(f"[{cfg.name}] skewed workgroups: prompt {P} + decode {N}, greedy and top-k")
    prompt = synth.prompt_ids(P, cfg.vocab_size, 21)
    eng = Engine(cfg, wd, P + N)

    def run(smp):
        import torch
        tokens = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
        last = torch.empty(cfg.vocab_size, dtype=torch.float32, device="cuda")
        first = eng.prefill(tokens, logits_out=last, smp=smp)
        out = torch.empty(N, dtype=torch.int32, device="cuda")
        logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
        eng.generate(first, N, out, logits, smp=smp)
        eng.sync()
        return int(first.item()), last.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy()

    greedy, topk = sampling(), sampling(50, 0.8, 2)
    ref = run(greedy)
    eng.reset()
    ref_k = run(topk)
    for level in (4, 16):
        eng.reset()
        eng.set_skew(level)
        got = run(greedy)
        eng.reset()
        got_k = run(topk)
        eng.set_skew(0)
        for a, b in ((ref, got), (ref_k, got_k)):
            assert a[0] == b[0] and np.array_equal(a[1], b[1]), f"skew {level}: prompt differs"
            assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3]), f"skew {level}: decode differs"
        say(f"  skew {level}: identical")
    eng.close()


def test_moe_long_context_over_synthetic_kv(torch_cuda, oracle_lib):
    """The 128-expert layer shape (2 layers) over 12,288 cached positions: both sides start from
    the same seeded synthetic K/V rows, then decode 3 steps. Each workgroup's chunk then holds 48
    K/V tiles (6 per wave, 3 batches), so the two passes of attention over 4 query heads each
    reload several batches."""
    import torch
    from hbm_bandwidth_bound_amd.kie import Engine
    cfg = synth.MOE_2L
    n, N = 12288, 3
    say(f"[{cfg.name}] {n} synthetic cached positions + decode {N}")
    wd = synth.make_weights_torch(cfg, 0, device="cuda")
    eng = Engine(cfg, wd, n + N)
    kd, vd = synth.synthetic_kv_torch(cfg, n, seed=7, device="cuda")
    kv = eng.kv_view()
    kv[:, 0, :, :n] = kd
    kv[:, 1, :, :n] = vd
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
    del wd, kd, vd, kv
    torch.cuda.empty_cache()
    oracle_lib.set_threads(16)
    try:
        om = oracle_lib.OracleModel(cfg, w, n + N)
        k, v = om.kv_view()
        k[:, :, :n] = kn
        v[:, :, :n] = vn
        z = om.record_routes(n + N)
        ref = om.run([tok0] + [int(t) for t in toks[:-1]], start_pos=n)
        om.stop_recording()
    finally:
        oracle_lib.set_threads(1)
    m = route_margin(z[n:n + N], cfg.n_experts_active)
    say(f"  smallest router margin {m:.2e}")
    assert m > ROUTE_MARGIN, "a routing decision is within the margin of a tie; pick another seed"
    worst, checked = check_steps(logits, ref, toks, label=cfg.name)
    say(f"  worst rel-L2 {worst:.3e}, greedy checked on {checked}/{N} steps")
    ko, vo = om.kv_view()
    ek = rel_l2(synth.bf16_bits_to_f32(kg_new[:, 0]), synth.bf16_bits_to_f32(ko[:, :, n:n + N]))
    ev = rel_l2(synth.bf16_bits_to_f32(kg_new[:, 1]), synth.bf16_bits_to_f32(vo[:, :, n:n + N]))
    say(f"  appended cache rows rel-L2 K {ek:.3e} V {ev:.3e}")
    assert ek <= 1e-3 and ev <= 1e-3


def test_moe_topk_matches_oracle(torch_cuda, oracle_lib):
    """Top-k sampling (k 50, T 0.8) on the mixture-of-experts program: the GPU's draw equals the
    oracle sampler's draw on the GPU's own logits at every step, and against the oracle's logits
    the candidate sets, probabilities and (away from ties) tokens agree."""
    import torch
    from hbm_bandwidth_bound_amd.kie import Engine, sampling
    from tests.gpu_util import check_topk_steps
    cfg = synth.SMALL_MOE
    w = synth.make_weights_np(cfg, 0)
    P, N, k, T, seed = 24, 12, 50, 0.8, 2
    say(f"[{cfg.name}] top-k {k}, T {T}: prompt {P} + decode {N}")
    eng = Engine(cfg, to_device(w), P + N)
    prompt = synth.prompt_ids(P, cfg.vocab_size, 3)
    smp = sampling(k, T, seed)
    first = eng.prefill(torch.tensor(prompt, dtype=torch.int32, device="cuda"), smp=smp)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
    eng.generate(first, N, out, logits, smp=smp)
    eng.sync()
    toks, logits = out.cpu().numpy(), logits.cpu().numpy()
    eng.close()
    om = oracle_lib.OracleModel(cfg, w, P + N)
    z = om.record_routes(P + N)
    om.run(prompt)
    ref = om.run([int(first.item())] + [int(t) for t in toks[:-1]], start_pos=P)
    om.stop_recording()
    assert route_margin(z, cfg.n_experts_active) > ROUTE_MARGIN
    tok_checked, set_checked = check_topk_steps(logits, ref, toks, k, T, seed, P, label=cfg.name)
    say(f"  token checks {tok_checked}/{N}, set checks {set_checked}/{N}")
    assert set_checked > 0
