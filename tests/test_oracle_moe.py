"""Pins of the oracle's mixture-of-experts layer (no GPU).

The pages only say that a mixture-of-experts model reads its routed experts' weights per token
(aikraft.ru «3000 токенов в секунду…», §02 and §04; agentlenshq.com, 《突破内存墙…》, opening
section). The router reading -- softmax over all experts, the n_experts_active largest, their
weights renormalised to sum to 1 -- is checked here against brute force and closed forms, and
the expert layer against cases that reduce to the dense feed-forward block and against a PyTorch
CPU rendition in fp64.
"""
import math

import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("E,A", [(128, 8), (16, 4), (8, 8), (5, 1)])
def test_router_against_brute_force(oracle_lib, E, A):
    rng = np.random.default_rng(E * 131 + A)
    for trial in range(20):
        z = (rng.standard_normal(E) * 0.9).astype(np.float32)
        if trial % 4 == 1:  # exact ties: the lower index ranks first
            z[rng.integers(0, E, E // 2)] = z[0]
        idx, w = oracle_lib.moe_route(z, A)
        want = sorted(range(E), key=lambda i: (-float(z[i]), i))[:A]
        assert list(idx) == want
        # weights: softmax over all E, restricted to the chosen, renormalised (fp64 closed form)
        ex = [math.exp(float(z[i]) - float(z.max())) for i in range(E)]
        Z = math.fsum(ex)
        p = [e / Z for e in ex]
        S = math.fsum(p[i] for i in want)
        for j, i in enumerate(want):
            assert w[j] == pytest.approx(p[i] / S, rel=1e-12)
        assert math.fsum(w) == pytest.approx(1.0, abs=1e-12)
        # ratios are exp of logit differences, whatever the normalisation
        assert w[0] / w[-1] == pytest.approx(math.exp(float(z[want[0]]) - float(z[want[-1]])), rel=1e-12)
        if A == E:  # every expert active: the weights are the full softmax
            assert np.allclose(np.asarray(w)[np.argsort(idx)], p, rtol=1e-12, atol=0)
        if A == 1:
            assert w[0] == 1.0


def _dense_to_moe(cfg, w, E, copies):
    """A mixture-of-experts copy of a dense model whose experts are `copies` of the dense FFN
    (expert e = copies[e] applied to the dense matrices: 'same' or a seeded perturbation)."""
    mcfg = cfg.scaled(name=cfg.name + "-as-moe", ffn_dim=0, n_experts=E, n_experts_active=0,
                      expert_ffn_dim=cfg.ffn_dim)
    mw = {k: v for k, v in w.items() if k not in ("w_gate", "w_up", "w_down")}
    mw["moe_gate"] = [np.stack([w["w_gate"][l]] * E) for l in range(cfg.n_layers)]
    mw["moe_up"] = [np.stack([w["w_up"][l]] * E) for l in range(cfg.n_layers)]
    mw["moe_down"] = [np.stack([w["w_down"][l]] * E) for l in range(cfg.n_layers)]
    mw["w_router"] = [synth._weights_bits_np((E, cfg.d_model), 3, 100 + l) for l in range(cfg.n_layers)]
    return mcfg, mw


def test_single_expert_equals_dense_ffn(oracle_lib):
    """E = 1, one active expert: its weight is exactly 1, so the layer is the dense SwiGLU block
    and every logit is bitwise the dense model's."""
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    mcfg, mw = _dense_to_moe(cfg, w, 1, None)
    mcfg = mcfg.scaled(n_experts_active=1)
    toks = synth.prompt_ids(12, cfg.vocab_size, 4)
    dense = oracle_lib.OracleModel(cfg, w, 16).run(toks)
    moe = oracle_lib.OracleModel(mcfg, mw, 16).run(toks)
    assert np.array_equal(dense, moe)


def test_identical_experts_reduce_to_dense(oracle_lib):
    """All experts equal to the dense FFN and 3 of 8 active: the renormalised weights sum to 1,
    so the output is the dense one up to rounding (without the renormalisation it would be
    scaled by the chosen experts' share of the softmax, ~0.4-0.6)."""
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    mcfg, mw = _dense_to_moe(cfg, w, 8, None)
    mcfg = mcfg.scaled(n_experts_active=3)
    toks = synth.prompt_ids(8, cfg.vocab_size, 5)
    dense = oracle_lib.OracleModel(cfg, w, 8).run(toks)
    moe = oracle_lib.OracleModel(mcfg, mw, 8).run(toks)
    assert rel_l2(moe, dense) <= 1e-5


def test_expert_permutation_invariance(oracle_lib):
    """Renumbering the experts (router rows and expert matrices together) changes nothing: the
    expert id that the router picks is the one whose matrices run."""
    cfg = synth.TINY_MOE
    w = synth.make_weights_np(cfg, 0)
    perm = np.random.default_rng(9).permutation(cfg.n_experts)
    pw = dict(w)
    for k in ("w_router", "moe_gate", "moe_up", "moe_down"):
        pw[k] = [np.ascontiguousarray(a[perm]) for a in w[k]]
    toks = synth.prompt_ids(10, cfg.vocab_size, 7)
    a = oracle_lib.OracleModel(cfg, w, 10).run(toks)
    b = oracle_lib.OracleModel(cfg, pw, 10).run(toks)
    assert np.array_equal(a, b)


def test_moe_incremental_decode_equals_full_recompute(oracle_lib):
    """KV-cached decode vs the whole-sequence pass, whose expert layer is written grouped by
    expert (each expert over the rows routed to it): the same sums in another order."""
    cfg = synth.TINY_MOE
    w = synth.make_weights_np(cfg, 0)
    toks = synth.prompt_ids(40, cfg.vocab_size, 1)
    m = oracle_lib.OracleModel(cfg, w, 40)
    inc = m.run(toks)
    full = m.full_recompute(toks)
    assert rel_l2(inc, full) <= 1e-5


def test_moe_ffn_against_torch_fp64(oracle_lib):
    """The expert layer for one input against PyTorch CPU routines in fp64 (softmax, topk, silu,
    matmul): routing identical, output within fp32 rounding."""
    import torch
    import torch.nn.functional as F
    cfg = synth.SMALL_MOE
    w = synth.make_weights_np(cfg, 0)
    m = oracle_lib.OracleModel(cfg, w, 4)
    rng = np.random.default_rng(11)
    for l in range(cfg.n_layers):
        u = rng.standard_normal(cfg.d_model).astype(np.float32)
        y, z = m.moe_ffn(l, u)

        def t(a):
            return torch.from_numpy(synth.bf16_bits_to_f32(np.asarray(a)).astype(np.float64))

        ut = torch.from_numpy(u.astype(np.float64))
        logits = t(w["w_router"][l]) @ ut
        assert np.allclose(z, logits.numpy(), rtol=1e-5, atol=1e-6)
        p = torch.softmax(logits, dim=0)
        top = torch.topk(p, cfg.n_experts_active)
        wt = top.values / top.values.sum()
        ref = torch.zeros(cfg.d_model, dtype=torch.float64)
        for j, e in enumerate(top.indices.tolist()):
            h = F.silu(t(w["moe_gate"][l][e]) @ ut) * (t(w["moe_up"][l][e]) @ ut)
            ref += wt[j] * (t(w["moe_down"][l][e]) @ h)
        assert rel_l2(y, ref.numpy()) <= 1e-5


def test_moe_active_bytes(oracle_lib):
    """Active weights of the 128-expert model: attention, router and 8 routed experts per layer,
    the LM head and one embedding row: 3.04 B parameters, 6.08 GB in bf16."""
    bm = oracle_lib.bytes_model
    act = bm.active_params(synth.MOE)
    assert act / 1e9 == pytest.approx(3.04, abs=0.005)
    assert 2 * act / 1e9 == pytest.approx(6.084, abs=0.001)
