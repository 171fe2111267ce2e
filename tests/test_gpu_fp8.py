"""8-bit weights on the GPU vs the CPU oracle, through the C ABI (needs an MI355X).

The 8-bit format is e4m3fn codes with one fp32 scale per matrix; both sides widen every code
exactly to fp32 and multiply the finished dot product by the matrix's scale, so the two differ by
the order of fp32 sums only, as in the bf16 path: logits are compared at every step (rel-L2
<= 1e-3), greedy tokens wherever the oracle's top-2 gap exceeds 0.05, the KV cache element-wise
(rel-L2 <= 1e-3); at the full 24-layer depth every vector is held to rel-L2(GPU, fp64) <=
rel-L2(oracle, fp64) + 1e-3 against the float64 reference, see compare(). The synthetic scales
differ per matrix, so a scale applied to the wrong matrix fails; one test fills the LM head with every finite code, so each code's widening on the GPU is
checked against the oracle's decoder. Prompts run through the matrix-core prompt pass
(`kie_prefill`), whose GEMMs widen the codes to bf16 as they read them.
"""
import ctypes as C

import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests import fp64_ref
from tests.gpu_util import check_against_fp64, check_steps, greedy_where_decided, rel_l2, say, to_device, top2_gap

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def compare(torch, oracle_lib, cfg, w, wd, P, N, seed, label, deep=False):
    """Prompt of P tokens, then N decode steps in one launch, against the oracle: logits at every
    step and the KV cache within rel-L2 1e-3, greedy tokens wherever the oracle's top-2 gap exceeds
    0.05. deep: a full-depth model, where two correct float32 renditions drift apart by more than
    1e-3 (bf16 rounding flips of K/V entries, amplified by later layers): every vector is then held
    to rel-L2(GPU, fp64) <= rel-L2(oracle, fp64) + 1e-3 against the float64 reference
    (tests/fp64_ref.py), the rule of every full-depth test."""
    from hbm_bandwidth_bound_amd.kie import Engine
    say(f"[{label}] prompt {P} + decode {N}")
    eng = Engine(cfg, wd, P + N)
    prompt = synth.prompt_ids(P, cfg.vocab_size, seed)
    tokens = torch.tensor(np.asarray(prompt, dtype=np.int32), device="cuda")
    last = torch.empty(cfg.vocab_size, dtype=torch.float32, device="cuda")
    first_t = eng.prefill(tokens, logits_out=last)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    logits = torch.empty((N, cfg.vocab_size), dtype=torch.float32, device="cuda")
    eng.generate(first_t, N, out, logits)
    eng.sync()
    first, last, toks, logits = int(first_t.item()), last.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy()
    kg = eng.kv_view().cpu().numpy().view(np.uint16)
    eng.close()
    decode_in = [first] + [int(t) for t in toks[:-1]]
    om = oracle_lib.OracleModel(cfg, w, P + N)
    ref_prompt = om.run(prompt)
    ref = om.run(decode_in, start_pos=P)
    ko, vo = om.kv_view()
    n = P + N
    f = synth.bf16_bits_to_f32
    if deep:
        say("  float64 reference ...")
        r64, k64, v64 = fp64_ref.Fp64Decoder(cfg, w).run(list(prompt) + decode_in)
        check_against_fp64(last, ref_prompt[-1], r64[P - 1], f"prompt position {P - 1}")
        for i in range(N):
            check_against_fp64(logits[i], ref[i], r64[P + i], f"decode position {P + i}")
        say(f"  greedy checked on {greedy_where_decided(toks, ref, label=label)}/{N} steps")
        check_against_fp64(f(kg[:, 0, :, :n]), f(ko[:, :, :n]), f(k64), "K cache")
        check_against_fp64(f(kg[:, 1, :, :n]), f(vo[:, :, :n]), f(v64), "V cache")
        return logits
    e = rel_l2(last, ref_prompt[-1])
    say(f"  prompt last-logits rel-L2 {e:.3e}")
    assert e <= 1e-3
    if top2_gap(ref_prompt[-1]) > 0.05:
        assert first == int(np.argmax(ref_prompt[-1]))
    worst, checked = check_steps(logits, ref, toks, tol=1e-3, label=label)
    say(f"  decode worst rel-L2 {worst:.3e}, greedy checked on {checked}/{N} steps")
    ek = rel_l2(f(kg[:, 0, :, :n]), f(ko[:, :, :n]))
    ev = rel_l2(f(kg[:, 1, :, :n]), f(vo[:, :, :n]))
    say(f"  cache rel-L2 K {ek:.3e} V {ev:.3e}")
    assert ek <= 1e-3 and ev <= 1e-3
    return logits


def test_fp8_prompt_then_decode(torch_cuda, oracle_lib):
    """d 512, 8 query / 4 KV heads of 64, FFN 1536 (3 tiles of 512 per row), vocabulary 4096:
    several tiles per unit, a ragged last batch, and the prompt pass on the matrix cores."""
    cfg = synth.TINY_FP8
    w = synth.make_weights_np(cfg, 0)
    compare(torch_cuda, oracle_lib, cfg, w, to_device(w), 40, 12, 1, cfg.name)


def test_fp8_every_code_widens_like_the_oracle(torch_cuda, oracle_lib):
    """LM head codes uniform over all 254 finite codes (both signs, subnormals, 448): the logits
    then weigh every code's value, and must match the oracle's decoder."""
    cfg = synth.TINY_FP8
    w = synth.make_weights_np(cfg, 2)
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 254, size=(cfg.vocab_size, cfg.d_model)).astype(np.uint8)
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)  # skip 0x7F (NaN); 0xFF is never drawn
    assert codes.max() == 0xFE and not np.any((codes & 0x7F) == 0x7F)
    assert len(np.unique(codes)) == 254
    w["lm_head"] = codes
    w["w_scale"] = w["w_scale"].copy()
    w["w_scale"][-1] = 2.0 ** -9
    compare(torch_cuda, oracle_lib, cfg, w, to_device(w), 6, 4, 3, "tiny-fp8-all-codes")


def test_fp8_subnormal_codes_widen_like_the_oracle(torch_cuda, oracle_lib):
    """LM head of subnormal codes only (m * 2^-9, both signs, and zeros): every logit is made of
    them, so a conversion that flushed them would give zeros."""
    cfg = synth.TINY_FP8
    w = synth.make_weights_np(cfg, 2)
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, size=(cfg.vocab_size, cfg.d_model)).astype(np.uint8)
    w["lm_head"] = ((codes & 7) | ((codes & 8) << 4)).astype(np.uint8)  # exponent field 0
    w["w_scale"] = w["w_scale"].copy()
    w["w_scale"][-1] = 4.0
    logits = compare(torch_cuda, oracle_lib, cfg, w, to_device(w), 6, 4, 3, "tiny-fp8-subnormal-codes")
    assert np.abs(logits).max() > 0.01


def test_fp8_1_6b_layer_shape(torch_cuda, oracle_lib):
    """The 1.6B shape (d 2048, 16/8 heads of 128, FFN 8192, vocabulary 32,768) cut to two layers,
    weights generated on the GPU (the integer encoder gives the oracle the same codes)."""
    cfg = synth.M1_6B_FP8_2L
    oracle_lib.set_threads(16)
    try:
        wd = synth.make_weights_torch(cfg, 0, device="cuda")
        w = synth.weights_torch_to_np(wd)
        wq1 = synth._weights_bits_np(synth.mat_shape(cfg, "wq"), 0, synth.tensor_index("wq", 1))
        assert np.array_equal(w["wq"][1], synth.fp8_codes_np(wq1))
        compare(torch_cuda, oracle_lib, cfg, w, wd, 12, 4, 1, cfg.name)
    finally:
        oracle_lib.set_threads(1)


def test_fp8_prompt_pass_two_chunks(torch_cuda, oracle_lib):
    """The matrix-core prompt pass with 8-bit weights (codes widened to bf16 as they are read, the
    matrix scales in the GEMM epilogues): the 1.6B shape cut to two layers with a 600-token prompt
    (a full 512-position chunk and a ragged one, split-K O and down projections), every prompt K/V
    row and the last prompt logits against the oracle, which runs the prompt position by position,
    at 1e-3 flat; then 3 decode steps."""
    cfg = synth.M1_6B_FP8_2L
    oracle_lib.set_threads(16)
    try:
        wd = synth.make_weights_torch(cfg, 0, device="cuda")
        w = synth.weights_torch_to_np(wd)
        compare(torch_cuda, oracle_lib, cfg, w, wd, 600, 3, 4, "1.6b-fp8-2l, prompt 600")
    finally:
        oracle_lib.set_threads(1)


def test_fp8_full_1_6b_model(torch_cuda, oracle_lib):
    """All 24 layers of the 1.6B model with 8-bit weights, in the launch configuration of the
    benchmark: a short prompt and two decode steps, every logit and the cache against the oracle
    and the float64 reference (the full-depth rule, see compare())."""
    cfg = synth.M1_6B_FP8
    oracle_lib.set_threads(16)
    try:
        wd = synth.make_weights_torch(cfg, 0, device="cuda")
        w = synth.weights_torch_to_np(wd)
        compare(torch_cuda, oracle_lib, cfg, w, wd, 4, 2, 5, cfg.name, deep=True)
    finally:
        oracle_lib.set_threads(1)


def test_fp8_8b_layer_shape(torch_cuda, oracle_lib):
    """The 8B shape (d 4096, 32/8 heads: 4 query heads per KV head, FFN 14,336 = 28 tiles of 512,
    vocabulary 128,256) cut to two layers."""
    cfg = synth.M8B_FP8.scaled(name="8b-fp8-2l", n_layers=2)
    oracle_lib.set_threads(16)
    try:
        wd = synth.make_weights_torch(cfg, 0, device="cuda")
        w = synth.weights_torch_to_np(wd)
        compare(torch_cuda, oracle_lib, cfg, w, wd, 6, 3, 2, cfg.name)
    finally:
        oracle_lib.set_threads(1)


def test_fp8_rejects_unsupported_configs(torch_cuda):
    """Refused on the host, before any launch: experts with 8-bit weights, rows that are not whole
    512-weight tiles, an unknown format, missing or non-finite scales."""
    from hbm_bandwidth_bound_amd import kie
    lib = kie.load()
    ok = synth.TINY_FP8
    assert lib.kie_packed_weight_bytes(C.byref(kie.make_config(ok, 64))) > 0
    bad = [synth.TINY_MOE.scaled(weight_format=1), synth.TINY.scaled(weight_format=1), ok.scaled(ffn_dim=1280),
           ok.scaled(weight_format=2)]
    for b in bad:
        assert lib.kie_packed_weight_bytes(C.byref(kie.make_config(b, 64))) == 0, b
    # at the 1.6B shape the 8-bit streams hold half the matrix bytes, plus the zero padding of the
    # QKV and O stages, where each wave's units fill half a batch (0.30 GB)
    b16 = lib.kie_packed_weight_bytes(C.byref(kie.make_config(synth.M1_6B, 64)))
    b8 = lib.kie_packed_weight_bytes(C.byref(kie.make_config(synth.M1_6B_FP8, 64)))
    emb = synth.M1_6B.vocab_size * synth.M1_6B.d_model * 2
    L, d = synth.M1_6B.n_layers, synth.M1_6B.d_model
    pad = L * (2 * d * d + d * d)  # QKV (4096 x 2048) and O (2048 x 2048) once more, as zeros
    assert b8 - emb == (b16 - emb) // 2 + pad
    wd = to_device(synth.make_weights_np(ok, 0))
    no_sc = {k: v for k, v in wd.items() if k != "w_scale"}
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(ok, no_sc, 64)
    assert ei.value.status == -1
    inf_sc = dict(wd, w_scale=np.full(ok.n_layers * 7 + 1, np.inf, dtype=np.float32))
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(ok, inf_sc, 64)
    assert ei.value.status == -1
