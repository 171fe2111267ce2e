"""Algorithmic bytes of the decode path (what one step must move), used for the roofline.

One decode step at position p reads every layer matrix and the LM head once (bf16, or 8-bit codes
and their scales), the norm
gains, one embedding row, the K and V rows of positions 0..p of every layer and KV head, and
writes the K and V rows of position p. In a mixture-of-experts layer the matrices read are the
attention's, the router's and those of the routed experts only. This is the pages' bytes-per-token model (aikraft.ru
«3000 токенов в секунду…», §02: tokens/s = effective bandwidth / active bytes) with the KV term
added, since the pages' bound leaves KV traffic out.
"""
from __future__ import annotations


def matrix_weights(m) -> int:
    """Weights of the layer matrices and the LM head one step reads. A mixture-of-experts layer
    reads its router and only the routed experts (n_experts_active of them)."""
    d, q, kv, f, V, L = m.d_model, m.n_heads * m.head_dim, m.n_kv_heads * m.head_dim, m.ffn_dim, m.vocab_size, m.n_layers
    if m.n_experts:
        ffn = m.n_experts * d + m.n_experts_active * 3 * m.expert_ffn_dim * d
    else:
        ffn = 3 * f * d
    return L * (q * d + 2 * kv * d + d * q + ffn) + V * d


def weight_bytes(m) -> int:
    """Weight bytes one step reads: the matrices (2 bytes a weight, or 1 with 8-bit weights plus
    their fp32 scales), the bf16 norm gains and one bf16 embedding row."""
    d, L = m.d_model, m.n_layers
    if getattr(m, "weight_format", 0) == 1:
        mats = matrix_weights(m) + 4 * (7 * L + 1)
    else:
        mats = 2 * matrix_weights(m)
    return mats + 2 * ((2 * L + 1) * d + d)


def kv_row_bytes(m) -> int:
    """K and V rows of one position across all layers and KV heads."""
    return 2 * m.n_layers * 2 * m.n_kv_heads * m.head_dim


def step_bytes(m, pos: int) -> int:
    return weight_bytes(m) + kv_row_bytes(m) * (pos + 1) + kv_row_bytes(m)


def launch_bytes(m, pos0: int, n_steps: int) -> int:
    """Bytes of n_steps decode steps at positions pos0 .. pos0 + n_steps - 1."""
    w = weight_bytes(m) * n_steps
    r = kv_row_bytes(m)
    # sum over s of (pos0 + s + 1) rows read + 1 row written
    reads = r * (n_steps * (pos0 + 1) + n_steps * (n_steps - 1) // 2)
    return w + reads + r * n_steps


def step_flops(m, pos: int) -> int:
    """Multiply-adds x 2 of one step: every weight once, plus QK and PV over pos+1 positions."""
    macs = matrix_weights(m) + 2 * m.n_layers * m.n_heads * m.head_dim * (pos + 1)
    return 2 * macs
