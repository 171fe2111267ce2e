"""Pins of the oracle's 8-bit weight format (no GPU).

The pages say that 8-bit weights halve the bytes a bandwidth-bound decoder reads per token, at
some cost in accuracy (aikraft.ru «3000 токенов в секунду…», §02; wink.run, 《GPU 算力越堆越高,
生成 token 为什么还是慢》, the section on what optimisations change), and fix no format. The oracle
reads it as e4m3fn codes with one fp32 scale per matrix. Pinned here: the code decoder against
PyTorch's own float8_e4m3fn type over all 256 codes, the 8-bit GEMV against an fp64 matrix product
of the decoded matrix, and the whole 8-bit model against the (already pinned) bf16 model whose
matrices are the decoded codes times power-of-two scales, which must agree bit for bit.
"""
import numpy as np
import pytest
import torch

from hbm_bandwidth_bound_amd import synth


def test_e4m3_decoder_matches_torch_for_every_code(oracle_lib):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle_lib.e4m3_to_f32(c) for c in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]  # the format's only NaNs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # closed forms: largest finite, smallest subnormal, one, negative zero
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert got[0x80] == 0.0 and np.signbit(got[0x80])


def test_generator_codes_match_torch_cast():
    bits = synth._weights_bits_np((1 << 16,), 0, 9)
    want = torch.from_numpy(synth.bf16_bits_to_f32(bits) * 128).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.fp8_codes_np(bits), want)


@pytest.mark.parametrize("rows,cols,scale", [(7, 512, 2.0 ** -7), (33, 1536, 0.01171875), (2, 4096, 3.0)])
def test_fp8_gemv_against_fp64_product(oracle_lib, rows, cols, scale):
    rng = np.random.default_rng(rows * cols)
    W = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
    W[(W & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    x = rng.standard_normal(cols).astype(np.float32)
    dec = torch.from_numpy(W).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = scale * (dec @ x.astype(np.float64))
    got = oracle_lib.gemv_e4m3(W, scale, x)
    # fp32 sum of cols products: relative to the sum of |terms|
    bound = 2 * cols * 2.0 ** -24 * scale * (np.abs(dec) @ np.abs(x).astype(np.float64))
    assert np.all(np.abs(got - want) <= bound + 1e-30)
    # the scale multiplies the finished sum
    assert np.array_equal(oracle_lib.gemv_e4m3(W, 2.0 * scale, x), 2.0 * got)


def _bf16_twin(cfg, w8, scales):
    """bf16 weights equal to scale * decoded codes (exact: 3 mantissa bits and power-of-two
    scales), for the same model in the bf16 format."""
    def bf16_of(codes, sc):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * float(sc)
        return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    wb = {k: v for k, v in w8.items() if k != "w_scale"}
    for l in range(cfg.n_layers):
        for m, name in enumerate(synth.LAYER_MATS):
            wb[name] = list(wb[name]) if l == 0 else wb[name]
            wb[name][l] = bf16_of(w8[name][l], scales[l * 7 + m])
    wb["lm_head"] = bf16_of(w8["lm_head"], scales[-1])
    # the twin really is exact
    for l in range(cfg.n_layers):
        for m, name in enumerate(synth.LAYER_MATS):
            back = torch.from_numpy(wb[name][l].view(np.int16)).view(torch.bfloat16).to(torch.float64)
            dec = torch.from_numpy(w8[name][l]).view(torch.float8_e4m3fn).to(torch.float64) * float(scales[l * 7 + m])
            assert torch.equal(back, dec)
    return wb


def test_fp8_model_equals_its_bf16_twin(oracle_lib):
    cfg = synth.TINY_FP8
    w8 = synth.make_weights_np(cfg, seed=4)
    # power-of-two scales that differ per matrix: a scale taken from the wrong matrix changes bits
    scales = np.array([2.0 ** -(5 + (i % 5)) for i in range(cfg.n_layers * 7 + 1)], dtype=np.float32)
    w8 = dict(w8, w_scale=scales)
    wb = _bf16_twin(cfg, w8, scales)
    m8 = oracle_lib.OracleModel(cfg, w8, max_seq=24)
    mb = oracle_lib.OracleModel(cfg.scaled(weight_format=0), wb, max_seq=24)
    toks = synth.prompt_ids(20, cfg.vocab_size, seed=5)
    l8 = m8.run(toks)
    lb = mb.run(toks)
    assert np.array_equal(l8, lb)
    assert np.array_equal(m8.kcache, mb.kcache) and np.array_equal(m8.vcache, mb.vcache)
    # and a scale moved to another matrix is seen
    bad = scales.copy()
    bad[[3, 4]] = bad[[4, 3]]
    assert not np.array_equal(oracle_lib.OracleModel(cfg, dict(w8, w_scale=bad), max_seq=24).run(toks[:3]), l8[:3])


def test_fp8_incremental_matches_full_recompute(oracle_lib):
    cfg = synth.TINY_FP8
    w8 = synth.make_weights_np(cfg, seed=6)
    m = oracle_lib.OracleModel(cfg, w8, max_seq=16)
    toks = synth.prompt_ids(12, cfg.vocab_size, seed=7)
    inc = m.run(toks)
    full = m.full_recompute(toks)
    scale = float(np.abs(full).max())
    assert np.max(np.abs(inc - full)) <= 1e-5 * scale


def test_fp8_model_is_close_to_the_bf16_model_it_was_encoded_from(oracle_lib):
    """With scale 2^-7 on every matrix the 8-bit model is the bf16 model rounded to 4 significant
    bits: logits move by about the rounding (2^-4 relative per weight), not more."""
    cfg = synth.TINY_FP8
    w8 = synth.make_weights_np(cfg, seed=8)
    w8["w_scale"] = np.full(cfg.n_layers * 7 + 1, 2.0 ** -7, dtype=np.float32)
    wb = synth.make_weights_np(cfg.scaled(weight_format=0), seed=8)
    toks = synth.prompt_ids(6, cfg.vocab_size, seed=9)
    l8 = oracle_lib.OracleModel(cfg, w8, max_seq=8).run(toks)
    lb = oracle_lib.OracleModel(cfg.scaled(weight_format=0), wb, max_seq=8).run(toks)
    rel = np.linalg.norm(l8 - lb) / np.linalg.norm(lb)
    assert 1e-3 < rel < 0.1


def test_fp8_rejected_with_experts(oracle_lib):
    cfg = synth.TINY_MOE.scaled(weight_format=1)
    w = synth.make_weights_np(synth.TINY_MOE, seed=1)
    w["w_scale"] = np.ones(cfg.n_layers * 7 + 1, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle_lib.OracleModel(cfg, w, max_seq=4).step(1)
