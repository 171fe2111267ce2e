"""Pins of the float64 reference decoder (tests/fp64_ref.py), on the CPU.

The reference is held against things outside itself: torch's float -> bfloat16 rounding and its
float8_e4m3fn decoding, the CPU oracle on the tiny model (two independent implementations of the
same decoder: they must agree to float32 rounding level), and its own batched run against the
same positions split into a prompt and a continuation over the handed-over cache. The bars
allow for the bf16 rounding of K and V: where an entry lies within float32 noise of a rounding
boundary the two implementations may round it to different neighbours (see fp64_ref).
"""
import numpy as np
import pytest

from hbm_bandwidth_bound_amd import synth
from tests import fp64_ref
from tests.gpu_util import rel_l2


def test_round_to_bf16_matches_torch():
    import torch
    rng = np.random.default_rng(5)
    x32 = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                          # exact ties between two bf16 neighbours (the low 16 bits are 0x8000)
                          ((rng.integers(0x3C00, 0x4400, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = fp64_ref.round_to_bf16(x32.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(fp64_ref.f64_to_bf16_bits(got), (want.astype(np.float32).view(np.uint32) >> 16))


def test_e4m3_values_match_torch():
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp64_ref._E4M3
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], want[~nan])


def test_matches_the_oracle_on_the_tiny_model(oracle_lib):
    """Float64 against float32 on a 24-token prompt. All but a handful of the bf16 K/V entries are
    identical (an entry within float32 noise of a rounding boundary may round to the other
    neighbour, a relative step of 2^-8). Step by step over the oracle's own cache, the logits
    agree to float32 rounding level (~5e-7) except where the step's own new row rounded an entry
    the other way (a flip moves the logits by ~1e-4); the whole run stays within 5e-4."""
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 0)
    toks = synth.prompt_ids(24, cfg.vocab_size, 1)
    om = oracle_lib.OracleModel(cfg, w, 24)
    ref32 = om.run(toks)
    ref = fp64_ref.Fp64Decoder(cfg, w)
    ref64, kn, vn = ref.run(toks)
    assert max(rel_l2(ref32[t], ref64[t]) for t in range(len(toks))) < 5e-4
    ko, vo = om.kv_view()
    for new, old in ((kn, ko), (vn, vo)):
        diff = np.count_nonzero(new != old[:, :, :24])
        assert diff <= 0.002 * new.size, diff
    errs = []
    for t in range(1, len(toks)):
        lg = ref.run(toks[t:t + 1], start_pos=t, k_prefix=ko[:, :, :t], v_prefix=vo[:, :, :t])[0]
        errs.append(rel_l2(ref32[t], lg[0]))
    errs = np.array(errs)
    assert errs.max() < 5e-4
    assert np.count_nonzero(errs < 2e-6) >= len(errs) - 3, errs


def test_gqa_and_moe_paths_match_the_oracle(oracle_lib):
    """The other head grouping and the mixture-of-experts feed-forward against the oracle."""
    for cfg in (synth.TINY_MOE, synth.TINY.scaled(name="tiny-mha", n_kv_heads=4)):
        w = synth.make_weights_np(cfg, 0)
        toks = synth.prompt_ids(10, cfg.vocab_size, 2)
        ref32 = oracle_lib.OracleModel(cfg, w, 10).run(toks)
        ref64 = fp64_ref.Fp64Decoder(cfg, w).run(toks)[0]
        assert max(rel_l2(ref32[t], ref64[t]) for t in range(10)) < 5e-4, cfg.name


def test_8bit_weights_match_the_oracle(oracle_lib):
    cfg = synth.TINY_FP8
    w = synth.make_weights_np(cfg, 0)
    toks = synth.prompt_ids(8, cfg.vocab_size, 3)
    ref32 = oracle_lib.OracleModel(cfg, w, 8).run(toks)
    ref64 = fp64_ref.Fp64Decoder(cfg, w).run(toks)[0]
    assert max(rel_l2(ref32[t], ref64[t]) for t in range(8)) < 5e-4


def test_handover_of_the_cache_equals_one_run():
    """Positions 0..9 in one run, and 0..5 then 6..9 over the first run's K/V rows: the same
    logits (up to the summation order of the batched products) and the same new rows."""
    cfg = synth.TINY
    w = synth.make_weights_np(cfg, 1)
    toks = synth.prompt_ids(10, cfg.vocab_size, 4)
    ref = fp64_ref.Fp64Decoder(cfg, w)
    full, kf, vf = ref.run(toks)
    a, ka, va = ref.run(toks[:6])
    b, kb, vb = ref.run(toks[6:], start_pos=6, k_prefix=ka, v_prefix=va)
    assert rel_l2(np.concatenate([a, b]), full) < 1e-13
    assert np.array_equal(np.concatenate([ka, kb], axis=2), kf)
    assert np.array_equal(np.concatenate([va, vb], axis=2), vf)
