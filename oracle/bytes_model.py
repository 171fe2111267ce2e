"""Bytes-per-token bound of batch-1 decoding (test infrastructure only).

The pages' model: in batch-1 decoding every active weight crosses the memory hierarchy once per
generated token, so tokens/s is the effective memory bandwidth divided by the active weight bytes
(aikraft.ru «3000 токенов в секунду…», §02 "Главный враг скорости…"; wink.run
《GPU 算力越堆越高,生成 token 为什么还是慢》, the 70B worked example). The pages ignore KV-cache
traffic; this model adds it as a separate term (K and V rows of every cached position are read,
one new row per layer is written) so that long-context runs are priced honestly.
"""
from __future__ import annotations


def weight_bytes_per_token(n_active_params: float, bytes_per_param: float) -> float:
    """Active weight bytes streamed per token (the pages' bound, KV ignored)."""
    return n_active_params * bytes_per_param


def tokens_per_second_bound(bandwidth_bytes_per_s: float, bytes_per_token: float) -> float:
    return bandwidth_bytes_per_s / bytes_per_token


def seconds_per_token(bytes_per_token: float, bandwidth_bytes_per_s: float) -> float:
    return bytes_per_token / bandwidth_bytes_per_s


def launch_overhead_bound(us_per_launch: float, launches_per_layer: int, n_layers: int):
    """Launch overhead per token (µs) and the tokens/s ceiling it alone imposes."""
    us = us_per_launch * launches_per_layer * n_layers
    return us, 1e6 / us


def arithmetic_intensity(bytes_per_weight: float) -> float:
    """FLOP per byte of a batch-1 GEMV: one multiply-add (2 FLOP) per weight."""
    return 2.0 / bytes_per_weight


# ------------------------------------------------------------------ decoder-specific counts

def dense_layer_params(cfg) -> int:
    d = cfg.d_model
    q = cfg.n_heads * cfg.head_dim
    kv = cfg.n_kv_heads * cfg.head_dim
    return d + q * d + 2 * kv * d + d * q + d + 3 * cfg.ffn_dim * d


def moe_layer_params(cfg, active: bool) -> int:
    d = cfg.d_model
    q = cfg.n_heads * cfg.head_dim
    kv = cfg.n_kv_heads * cfg.head_dim
    e = cfg.n_experts_active if active else cfg.n_experts
    return d + q * d + 2 * kv * d + d * q + d + cfg.n_experts * d + e * 3 * cfg.expert_ffn_dim * d


def total_params(cfg) -> int:
    """All stored parameters: embedding, LM head, final norm and every layer."""
    per = moe_layer_params(cfg, active=False) if cfg.n_experts else dense_layer_params(cfg)
    return 2 * cfg.vocab_size * cfg.d_model + cfg.d_model + cfg.n_layers * per


def active_params(cfg) -> int:
    """Parameters read for one token: all layers (routed experts only), final norm, LM head and
    one embedding row."""
    per = moe_layer_params(cfg, active=True) if cfg.n_experts else dense_layer_params(cfg)
    return cfg.vocab_size * cfg.d_model + cfg.d_model + cfg.d_model + cfg.n_layers * per


def kv_bytes_per_position(cfg, bytes_per_elem: int = 2) -> int:
    """K and V rows of one position over all layers."""
    return cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * bytes_per_elem


def decode_step_bytes(cfg, pos: int, bytes_per_param: int = 2) -> int:
    """Bytes one decode step at position `pos` must move: active weights, the K/V rows of
    positions 0..pos read by attention, and the new K/V row written."""
    kvp = kv_bytes_per_position(cfg)
    return active_params(cfg) * bytes_per_param + kvp * (pos + 1) + kvp


def mean_decode_bytes(cfg, prompt_len: int, steps: int) -> float:
    """Mean of decode_step_bytes over the decode positions prompt_len .. prompt_len+steps-1."""
    tot = sum(decode_step_bytes(cfg, prompt_len + s) for s in range(steps))
    return tot / steps


def decode_step_bytes_8bit(cfg, pos: int) -> int:
    """decode_step_bytes for a model whose layer matrices and LM head are 8-bit codes: one byte per
    matrix weight and one fp32 scale per matrix (seven per layer and the LM head's), while the norm
    gains, the embedding row and the KV cache stay bf16 (the pages: 8-bit weights halve the bytes
    a bandwidth-bound decoder streams; aikraft.ru «3000 токенов в секунду…», §02)."""
    d = cfg.d_model
    gains = (2 * cfg.n_layers + 1) * d        # attention and FFN norms per layer, final norm
    matrices = active_params(cfg) - gains - d  # everything else but the one embedding row
    kvp = kv_bytes_per_position(cfg)
    return matrices + 4 * (7 * cfg.n_layers + 1) + 2 * (gains + d) + kvp * (pos + 1) + kvp
