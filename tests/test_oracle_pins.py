"""Pins of the CPU oracle to what the pages and mathematics fix (no GPU).

Each test checks the oracle against something other than itself: numbers printed on the pages,
closed forms, invariants, special cases that reduce to a textbook or library routine, brute force
on tiny inputs, or exact results within a proven error bound.
"""
import json
import math
import os

import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bf16_bits(x):
    """fp32 array -> bf16 bits (RNE) by NumPy, used only to build test inputs."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# ------------------------------------------------------------------ byte model vs the pages

@pytest.fixture(scope="module")
def pages():
    with open(os.path.join(GOLDEN, "pages_closed_forms.json")) as f:
        return json.load(f)


def test_light_speed_bounds_match_pages(oracle_lib, pages):
    bm = oracle_lib.bytes_model
    g = pages["light_speed_8xH200"]
    agg = g["per_card_TBps"] * g["cards"] * g["realistic_fraction"]
    assert agg == pytest.approx(g["aggregate_TBps"], rel=0.002)
    b = bm.weight_bytes_per_token(g["params"], g["bytes_per_param"])
    assert b == pytest.approx(g["weight_GB"] * 1e9)
    assert bm.tokens_per_second_bound(g["aggregate_TBps"] * 1e12, b) == pytest.approx(g["tok_s"], rel=g["rel_tol"])
    for key in ("light_speed_8xMI300X", "moe_fp8_4B_active", "moe_fp4_32B_active"):
        g = pages[key]
        b = bm.weight_bytes_per_token(g["params"], g["bytes_per_param"])
        assert bm.tokens_per_second_bound(g["aggregate_TBps"] * 1e12, b) == pytest.approx(g["tok_s"], rel=g["rel_tol"])


def test_70b_worked_example(oracle_lib, pages):
    bm = oracle_lib.bytes_model
    g = pages["h100_70B_16bit"]
    b = bm.weight_bytes_per_token(g["params"], g["bytes_per_param"])
    assert b == pytest.approx(g["weight_GB"] * 1e9)
    ms = 1e3 * bm.seconds_per_token(b, g["bandwidth_TBps"] * 1e12)
    assert ms == pytest.approx(g["ms_per_token"], rel=g["rel_tol"])
    assert bm.tokens_per_second_bound(g["bandwidth_TBps"] * 1e12, b) == pytest.approx(g["tok_s"], rel=0.01)
    g8 = pages["h100_70B_8bit"]
    b8 = bm.weight_bytes_per_token(g8["params"], g8["bytes_per_param"])
    assert b8 == pytest.approx(g8["weight_GB"] * 1e9)
    assert bm.tokens_per_second_bound(g8["bandwidth_TBps"] * 1e12, b8) == pytest.approx(g8["tok_s"], rel=g8["rel_tol"])


def test_launch_overhead_and_budget(oracle_lib, pages):
    bm = oracle_lib.bytes_model
    for key in ("launch_overhead_10_kernels", "launch_overhead_5_kernels"):
        g = pages[key]
        us, tok = bm.launch_overhead_bound(g["us_per_launch"], g["kernels_per_layer"], g["layers"])
        assert us == pytest.approx(g["overhead_us"], rel=g["rel_tol"])
        assert tok == pytest.approx(g["tok_s"], rel=g["rel_tol"])
    g = pages["per_token_budget"]
    assert 1e6 / g["tok_s"] == pytest.approx(g["us_per_token"], rel=g["rel_tol"])
    assert g["us_lost_per_layer"] * g["layers"] / (1e6 / g["tok_s"]) == pytest.approx(g["budget_fraction"], rel=0.01)


def test_intensity_and_ridges(oracle_lib, pages):
    bm = oracle_lib.bytes_model
    g = pages["arithmetic_intensity"]
    assert bm.arithmetic_intensity(2) == g["fp16"]
    assert bm.arithmetic_intensity(1) == g["fp8"]
    assert bm.arithmetic_intensity(0.5) == g["fp4"]
    r = pages["ridge_points"]
    assert r["peak_TFLOPS"] / r["h100_TBps"] == pytest.approx(r["h100_ridge"], rel=r["rel_tol"])
    assert r["peak_TFLOPS"] / r["h200_TBps"] == pytest.approx(r["h200_ridge"], rel=r["rel_tol"])
    a = pages["agent_workflow"]
    assert a["tokens"] / a["slow_tok_s"] / 60 == pytest.approx(a["slow_minutes_approx"], rel=0.05)
    assert a["tokens"] / a["fast_tok_s"] < a["fast_seconds_max"]


def test_config_sizes_match_shape_notes(oracle_lib):
    """Parameter and KV sizes of the named configurations: ~1.644B params (1.6B), ~16.06 GB (8B),
    ~61.06 GB (MoE), ~3.25 GB of bf16 KV for 33,024 positions of the 1.6B model."""
    bm = oracle_lib.bytes_model
    assert bm.total_params(synth.M1_6B) == 1_644_267_520
    assert 2 * bm.total_params(synth.M8B) / 1e9 == pytest.approx(16.06, abs=0.005)
    assert 2 * bm.total_params(synth.MOE) / 1e9 == pytest.approx(61.06, abs=0.005)
    assert bm.kv_bytes_per_position(synth.M1_6B) * 33024 / 1e9 == pytest.approx(3.25, abs=0.005)
    # one decode step of the 1.6B model: 3,154,321,408 weight bytes plus 98,304 B per KV position
    assert bm.decode_step_bytes(synth.M1_6B, 0) - 2 * bm.kv_bytes_per_position(synth.M1_6B) == 3_154_321_408
    assert bm.kv_bytes_per_position(synth.M1_6B) == 98_304
    # tiny: every parameter count by hand: 2*4096*256 + 256 + 2*(2*256 + 3*256*... )
    t = synth.TINY
    per_layer = 2 * 256 + 256 * 256 + 2 * 128 * 256 + 256 * 256 + 3 * 1024 * 256
    assert bm.total_params(t) == 2 * 4096 * 256 + 256 + 2 * per_layer


# ------------------------------------------------------------------ building blocks

def test_gemv_orientation_and_higham_bound(oracle_lib):
    rng = np.random.default_rng(5)
    # orientation: a permutation matrix P with P[r][perm[r]] = 1 must give y = x[perm]
    n = 37
    perm = rng.permutation(n)
    P = np.zeros((n, n), dtype=np.uint16)
    P[np.arange(n), perm] = 0x3F80
    x = rng.standard_normal(n).astype(np.float32)
    assert np.array_equal(oracle_lib.gemv(P, x), x[perm])
    # non-square: y has `rows` entries built from row r of W
    W = bf16_bits(rng.standard_normal((5, 300)).astype(np.float32))
    x = rng.standard_normal(300).astype(np.float32)
    y = oracle_lib.gemv(W, x)
    wf = synth.bf16_bits_to_f32(W).astype(np.float64)
    exact = wf @ x.astype(np.float64)  # products of bf16 x fp32 are exact in fp64
    K = 300
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    bound = gamma * (np.abs(wf) @ np.abs(x.astype(np.float64)))
    assert np.all(np.abs(y - exact) <= bound)
    # large K as in the down projection
    K = 8192
    W = bf16_bits(rng.standard_normal((4, K)).astype(np.float32) * 0.02)
    x = rng.standard_normal(K).astype(np.float32)
    y = oracle_lib.gemv(W, x)
    wf = synth.bf16_bits_to_f32(W).astype(np.float64)
    gamma = K * u / (1 - K * u)
    assert np.all(np.abs(y - wf @ x.astype(np.float64)) <= gamma * (np.abs(wf) @ np.abs(x.astype(np.float64))))


def test_rmsnorm_closed_forms(oracle_lib):
    eps = 1e-6
    for c in (0.5, 3.0, -2.0):
        x = np.full(256, c, dtype=np.float32)
        g = bf16_bits(np.linspace(0.5, 2.0, 256).astype(np.float32))
        u = oracle_lib.rmsnorm(x, g, eps)
        expect = synth.bf16_bits_to_f32(g).astype(np.float64) * c / math.sqrt(c * c + eps)
        assert np.allclose(u, expect, rtol=3e-7, atol=0)
    # unit gains: the output has mean square 1 (up to eps) for any input
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(2048) * 7).astype(np.float32)
    u = oracle_lib.rmsnorm(x, np.full(2048, 0x3F80, np.uint16), eps)
    assert float(np.mean(u.astype(np.float64) ** 2)) == pytest.approx(1.0, rel=1e-5)
    # the output direction is the input's
    assert np.allclose(u / np.linalg.norm(u), x / np.linalg.norm(x), atol=1e-6)


def test_rope_angle_identity_norm_and_relative_position(oracle_lib):
    hd, theta = 64, 10000.0
    rng = np.random.default_rng(2)
    y = rng.standard_normal(hd).astype(np.float32)
    assert np.array_equal(oracle_lib.rope(y, 0, theta), y)  # position 0 is the identity
    # a unit vector in pair i is rotated counter-clockwise by pos * theta^(-2i/hd)
    for i in (0, 1, 5, 31):
        for pos in (1, 7, 1000):
            e = np.zeros(hd, np.float32)
            e[i] = 1.0
            r = oracle_lib.rope(e, pos, theta)
            phi = pos * theta ** (-2.0 * i / hd)
            assert r[i] == pytest.approx(math.cos(phi), abs=1e-6)
            assert r[i + hd // 2] == pytest.approx(math.sin(phi), abs=1e-6)
            others = np.delete(r, [i, i + hd // 2])
            assert np.all(others == 0)
    # pair norms are preserved
    r = oracle_lib.rope(y, 123, theta)
    half = hd // 2
    n0 = np.hypot(y[:half].astype(np.float64), y[half:].astype(np.float64))
    n1 = np.hypot(r[:half].astype(np.float64), r[half:].astype(np.float64))
    assert np.allclose(n0, n1, rtol=1e-6)
    # <R_m q, R_n k> depends on m - n only (RoFormer, Su et al. 2021)
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    a = float(np.dot(oracle_lib.rope(q, 10, theta).astype(np.float64), oracle_lib.rope(k, 3, theta)))
    b = float(np.dot(oracle_lib.rope(q, 107, theta).astype(np.float64), oracle_lib.rope(k, 100, theta)))
    assert a == pytest.approx(b, rel=1e-5, abs=1e-5)


def test_attention_special_cases(oracle_lib):
    rng = np.random.default_rng(3)
    hd = 64
    # one position returns V exactly
    q = rng.standard_normal(hd).astype(np.float32)
    K = bf16_bits(rng.standard_normal((1, hd)))
    V = bf16_bits(rng.standard_normal((1, hd)))
    out, p = oracle_lib.attend(q, K, V)
    assert np.array_equal(out, synth.bf16_bits_to_f32(V[0]))
    assert p[0] == 1.0
    # equal scores (q = 0) give the mean of V
    n = 50
    K = bf16_bits(rng.standard_normal((n, hd)))
    V = bf16_bits(rng.standard_normal((n, hd)))
    out, p = oracle_lib.attend(np.zeros(hd, np.float32), K, V)
    assert np.allclose(out, synth.bf16_bits_to_f32(V).astype(np.float64).mean(0), atol=1e-6)
    # a dominant key selects its value
    K = np.zeros((n, hd), np.uint16)
    K[17] = bf16_bits(np.full(hd, 4.0, np.float32))
    out, p = oracle_lib.attend(np.full(hd, 4.0, np.float32), K, V)
    assert np.argmax(p) == 17 and p[17] > 1 - 1e-12


@pytest.mark.parametrize("n", [1, 7, 1024, 33024])
def test_softmax_rows_sum_to_one(oracle_lib, n):
    rng = np.random.default_rng(n)
    hd = 128
    q = (rng.standard_normal(hd) * 3).astype(np.float32)
    K = bf16_bits(rng.standard_normal((n, hd)))
    V = bf16_bits(rng.standard_normal((n, hd)))
    _, p = oracle_lib.attend(q, K, V)
    assert abs(math.fsum(p) - 1.0) <= 1e-6
    # and p is the softmax of the scaled scores (fp64 reference of the probabilities)
    s = (synth.bf16_bits_to_f32(K).astype(np.float64) @ q.astype(np.float64)) / math.sqrt(hd)
    ref = np.exp(s - s.max())
    ref /= ref.sum()
    assert np.allclose(p, ref, rtol=2e-5, atol=1e-12)


def test_silu(oracle_lib):
    from scipy.special import expit
    assert oracle_lib.silu(0.0) == 0.0
    for g in (-20.0, -3.5, -0.1, 0.25, 1.0, 6.0, 30.0):
        assert oracle_lib.silu(g) == pytest.approx(g * expit(g), rel=1e-6, abs=1e-30)


def test_bf16_round_to_nearest_even(oracle_lib):
    # 1 + 2^-8 is the midpoint between bf16 1.0 and 1.0078125: ties go to the even mantissa (1.0)
    assert oracle_lib.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint between 1.0078125 (odd) and 1.015625 (even): rounds up
    assert oracle_lib.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle_lib.f32_to_bf16(-2.0) == 0xC000
    for b in (0x0000, 0x3F80, 0x4049, 0xBF00, 0x7F7F):
        assert oracle_lib.f32_to_bf16(oracle_lib.bf16_to_f32(b)) == b


# ------------------------------------------------------------------ sampling

def test_splitmix64_published_values(oracle_lib):
    # SplitMix64 started from state 0: the generator adds the golden gamma and mixes; its first
    # three outputs are the widely published test vector below.
    gamma = 0x9E3779B97F4A7C15
    outs = [oracle_lib.splitmix64((i * gamma) % 2 ** 64) for i in range(3)]
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    us = [oracle_lib.uniform(2, p) for p in range(1000)]
    assert min(us) >= 0.0 and max(us) < 1.0
    assert abs(np.mean(us) - 0.5) < 0.05
    assert all(abs(u * 2 ** 24 - round(u * 2 ** 24)) == 0 for u in us)


def test_topk_against_brute_force(oracle_lib):
    rng = np.random.default_rng(7)
    V = 4096
    logits = (rng.standard_normal(V) * 2).astype(np.float32)
    logits[100] = logits[200] = logits.max() + 1  # a tie at the top: lower index first
    for k, T, seed, pos in ((50, 0.8, 2, 1024), (1, 0.8, 2, 5), (5, 1.0, 9, 0), (V, 1.3, 1, 77)):
        tok, idx, p, u = oracle_lib.topk_sample(logits, k, T, seed, pos)
        z = logits / np.float32(T)
        order = np.lexsort((np.arange(V), -z.astype(np.float64)))  # z desc, then index asc
        assert np.array_equal(idx, order[:k])
        e = np.exp(z[order[:k]].astype(np.float64) - float(z[order[0]]))
        assert np.allclose(p, e / e.sum(), rtol=1e-12)
        assert abs(math.fsum(p) - 1.0) <= 1e-12
        assert u == oracle_lib.uniform(seed, pos)
        j = int(np.searchsorted(np.cumsum(p), u, side="right"))
        assert tok == order[:k][min(j, k - 1)]
    assert idx is not None
    # k = 1 is greedy
    for s in range(5):
        lg = rng.standard_normal(V).astype(np.float32)
        assert oracle_lib.topk_sample(lg, 1, 0.8, s, s)[0] == oracle_lib.argmax(lg) == int(np.argmax(lg))
    # ties in argmax go to the lowest index
    lg = np.zeros(V, np.float32)
    lg[[9, 3000]] = 1.0
    assert oracle_lib.argmax(lg) == 9


# ------------------------------------------------------------------ whole decoder

@pytest.fixture(scope="module")
def tiny_model(oracle_lib):
    w = synth.make_weights_np(synth.TINY, 0)
    return w


def test_incremental_decode_equals_full_recompute(oracle_lib, tiny_model):
    """KV-cached incremental decode vs a brute-force causal pass over the whole sequence
    (tiny config, 64-token prompt + 32 greedy steps)."""
    cfg = synth.TINY
    prompt = synth.prompt_ids(64, cfg.vocab_size, 1)
    m = oracle_lib.OracleModel(cfg, tiny_model, 96)
    inc = [m.step(int(t)) for t in prompt]
    toks = list(prompt)
    for _ in range(32):
        toks.append(oracle_lib.argmax(inc[-1]))
        if len(toks) < 96:
            inc.append(m.step(toks[-1]))
    inc = np.stack(inc)
    full = oracle_lib.full_recompute(m, toks[:inc.shape[0]])
    assert rel_l2(inc, full) <= 1e-6
    assert np.array_equal(inc, full)  # same per-element arithmetic: bitwise equal
    # causality: changing a later token leaves earlier logits untouched
    toks2 = list(toks[:inc.shape[0]])
    toks2[50] = (toks2[50] + 1) % cfg.vocab_size
    full2 = oracle_lib.full_recompute(m, toks2)
    assert np.array_equal(full2[:50], full[:50])
    assert not np.array_equal(full2[50], full[50])


def test_gqa_equals_mha_with_repeated_kv_heads(oracle_lib, tiny_model):
    """Grouped-query attention reads KV head h // (nq/nkv): an MHA model whose K/V projections
    repeat each KV head for its group of query heads must give the same logits."""
    cfg = synth.TINY
    G = cfg.n_heads // cfg.n_kv_heads
    hd = cfg.head_dim
    mha_cfg = cfg.scaled(n_kv_heads=cfg.n_heads)
    w2 = dict(tiny_model)
    for name in ("wk", "wv"):
        w2[name] = [np.repeat(m.reshape(cfg.n_kv_heads, hd, cfg.d_model), G, axis=0).reshape(cfg.n_heads * hd, -1)
                    for m in tiny_model[name]]
    prompt = synth.prompt_ids(20, cfg.vocab_size, 3)
    a = oracle_lib.OracleModel(cfg, tiny_model, 32).run(prompt)
    b = oracle_lib.OracleModel(mha_cfg, w2, 32).run(prompt)
    assert np.array_equal(a, b)


def test_thread_split_is_bitwise_identical(oracle_lib, tiny_model):
    cfg = synth.TINY
    prompt = synth.prompt_ids(12, cfg.vocab_size, 4)
    oracle_lib.set_threads(1)
    a = oracle_lib.OracleModel(cfg, tiny_model, 16).run(prompt)
    oracle_lib.set_threads(4)
    b = oracle_lib.OracleModel(cfg, tiny_model, 16).run(prompt)
    oracle_lib.set_threads(1)
    assert np.array_equal(a, b)


def test_against_torch_cpu_library_rendition(oracle_lib, tiny_model):
    """The decoder written with PyTorch CPU library routines (rms_norm, scaled_dot_product_attention
    with its causal mask and 1/sqrt(hd) scale, silu, matmul) in fp32 over the whole sequence: the
    two fp32 renditions agree to 1e-6 in logits. The rendition runs on one thread: the thread count
    changes the library's summation order, and where that moves a key or value across a bf16
    rounding boundary, the positions after it differ by up to ~1e-5."""
    import torch
    import torch.nn.functional as F
    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        ref, got = _torch_rendition(oracle_lib, tiny_model, torch, F)
    finally:
        torch.set_num_threads(threads)
    assert rel_l2(got, ref) <= 1e-6
    assert np.array_equal(got.argmax(1), ref.argmax(1))


def _torch_rendition(oracle_lib, tiny_model, torch, F):
    cfg = synth.TINY
    d, hd, nq, nkv = cfg.d_model, cfg.head_dim, cfg.n_heads, cfg.n_kv_heads

    def t(a):
        return torch.from_numpy(synth.bf16_bits_to_f32(np.asarray(a)).copy())

    prompt = synth.prompt_ids(48, cfg.vocab_size, 6)
    n = len(prompt)
    pos = torch.arange(n, dtype=torch.float64)
    freq = cfg.rope_theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * freq[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()

    def rope(x):  # x [n, heads, hd]; rotate-half pairing
        a, b = x[..., : hd // 2], x[..., hd // 2:]
        c, s = cos[:, None, :], sin[:, None, :]
        return torch.cat([a * c - b * s, b * c + a * s], dim=-1)

    x = t(tiny_model["embed"])[torch.from_numpy(prompt.astype(np.int64))]
    for l in range(cfg.n_layers):
        u = F.rms_norm(x, (d,), weight=t(tiny_model["attn_norm"][l]), eps=cfg.rms_eps)
        q = rope((u @ t(tiny_model["wq"][l]).T).view(n, nq, hd))
        k = rope((u @ t(tiny_model["wk"][l]).T).view(n, nkv, hd))
        v = (u @ t(tiny_model["wv"][l]).T).view(n, nkv, hd)
        k = k.to(torch.bfloat16).float()
        v = v.to(torch.bfloat16).float()
        k = k.repeat_interleave(nq // nkv, dim=1)
        v = v.repeat_interleave(nq // nkv, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True)
        x = x + o.transpose(0, 1).reshape(n, nq * hd) @ t(tiny_model["wo"][l]).T
        u = F.rms_norm(x, (d,), weight=t(tiny_model["ffn_norm"][l]), eps=cfg.rms_eps)
        h = F.silu(u @ t(tiny_model["w_gate"][l]).T) * (u @ t(tiny_model["w_up"][l]).T)
        x = x + h @ t(tiny_model["w_down"][l]).T
    u = F.rms_norm(x, (d,), weight=t(tiny_model["final_norm"]), eps=cfg.rms_eps)
    ref = (u @ t(tiny_model["lm_head"]).T).numpy()
    return ref, oracle_lib.OracleModel(cfg, tiny_model, n).run(prompt)


def test_gemv_order_is_a_rounding_level_variant(oracle_lib):
    """The descending-order GEMV is the same sum: on the tiny model the two renditions agree to
    ~1e-6 in logits, far inside the 1e-3 bar (at 24 layers the same two renditions drift to ~2e-3,
    which is why the full-size GPU test measures that drift and allows twice it)."""
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    prompt = synth.prompt_ids(24, cfg.vocab_size, 1)
    a = oracle_lib.OracleModel(cfg, w, 24).run(prompt)
    oracle_lib.set_gemv_order(True)
    try:
        b = oracle_lib.OracleModel(cfg, w, 24).run(prompt)
        W = synth.bf16_bits_to_f32(w["lm_head"][:64]).astype(np.float32)
        x = np.linspace(-1, 1, cfg.d_model).astype(np.float32)
        y_desc = oracle_lib.gemv(w["lm_head"][:64], x)
    finally:
        oracle_lib.set_gemv_order(False)
    y_asc = oracle_lib.gemv(w["lm_head"][:64], x)
    exact = W.astype(np.float64) @ x.astype(np.float64)
    # both orders are within the fp32 summation bound of the exact sum, and they differ
    bound = 64 * np.finfo(np.float32).eps * (np.abs(W.astype(np.float64)) @ np.abs(x.astype(np.float64)))
    assert np.all(np.abs(y_asc - exact) <= bound) and np.all(np.abs(y_desc - exact) <= bound)
    assert not np.array_equal(y_asc, y_desc)
    spread = np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b.astype(np.float64))
    assert 0 < spread < 1e-4


def test_8bit_bytes_halve_the_weight_stream(oracle_lib):
    """The pages: 8-bit weights halve the bytes a bandwidth-bound decoder streams per token. With
    the KV rows set aside, the 8-bit model's bytes are half the bf16 model's, up to the bf16 norm
    gains and embedding row and the per-matrix scales (below 0.1% at these shapes)."""
    from hbm_bandwidth_bound_amd import synth
    bm = oracle_lib.bytes_model
    for m in (synth.M1_6B, synth.M8B):
        kv = bm.kv_bytes_per_position(m) * 2
        b16 = bm.decode_step_bytes(m, 0) - kv
        b8 = bm.decode_step_bytes_8bit(m, 0) - kv
        assert abs(b8 / b16 - 0.5) < 1e-3, (m.name, b8 / b16)
        assert b8 > b16 / 2  # the bf16 pieces and the scales only add
