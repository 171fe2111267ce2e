"""The decoder in float64 with NumPy: the reference the full-depth parity tests measure distances to.

Test infrastructure only, written independently of the CPU oracle (``oracle/``, C, float32) and of
the GPU kernels: it imports neither. It computes the same pre-RMSNorm decoder (RoPE on
rotate-half pairs, grouped-query attention, SwiGLU, untied LM head) from the bf16 weights (or
e4m3fn codes times their matrix scale) with every product, sum, norm, softmax and rotation in
float64, so its own rounding error (~1e-16 relative per operation) is negligible next to that of a
float32 rendition. The one rounding it keeps is the model's: the K and V rows are rounded to bf16
(to nearest, ties to even) before attention reads them, as the configuration's bf16 KV cache
requires.

Why it exists. At 24 layers the decoder amplifies float32 rounding differences: where a K or V
entry lies within float32 noise of a bf16 rounding boundary, two correct float32 renditions round
it to different neighbours (a relative step of 2^-8), and later layers carry the difference on.
Two float32 renditions (the oracle and the GPU) can then differ by more than 1e-3 while both are
within the same distance of the exact value. Measuring both against this float64 rendition
separates an arithmetic error (the GPU far from the exact value) from that amplified rounding
noise (both about equally far from it).

A run is ``T`` teacher-forced positions start_pos .. start_pos + T - 1 processed together (each
layer's weights are widened once per run), after a prefix of cached K/V rows [0, start_pos) that
the caller hands over (bf16 bits, e.g. another implementation's cache), or none.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 or int16 arrays) -> their exact float64 values."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (8 significant bits, ties to even), returned as float64.
    One rounding from the float64 value. The values here are far from bf16's range limits."""
    m, e = np.frexp(x)                    # x = m * 2^e with 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)  # np.round rounds halves to even


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are exactly bf16 already (as produced by round_to_bf16)."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _e4m3_values() -> np.ndarray:
    """Value of each of the 256 OCP E4M3 ("fn") codes: sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN; no infinities."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_E4M3 = _e4m3_values()
_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


class Fp64Decoder:
    """cfg: n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size, rms_eps,
    rope_theta (and optionally n_experts, n_experts_active, expert_ffn_dim, weight_format).
    weights: the arrays both implementations are built from (bf16 bits as uint16/int16; e4m3fn
    codes as uint8 with ``w_scale`` [n_layers * 7 + 1] when weight_format == 1)."""

    def __init__(self, cfg, weights):
        self.cfg = cfg
        self.w = weights
        self.w8 = int(getattr(cfg, "weight_format", 0)) == 1

    # ------------------------------------------------------------------ weights in float64
    def _mat(self, name: str, layer=None) -> np.ndarray:
        a = self.w[name] if layer is None else self.w[name][layer]
        if self.w8 and (name in _MATS or name == "lm_head"):
            idx = self.cfg.n_layers * 7 if name == "lm_head" else layer * 7 + _MATS.index(name)
            return _E4M3[np.asarray(a, dtype=np.uint8)] * float(np.float32(self.w["w_scale"][idx]))
        return bf16_bits_to_f64(a)

    def _gain(self, name: str, layer=None) -> np.ndarray:
        return bf16_bits_to_f64(self.w[name] if layer is None else self.w[name][layer])

    # ------------------------------------------------------------------ the decoder's steps
    def rmsnorm(self, X: np.ndarray, g: np.ndarray) -> np.ndarray:
        """Each row x of X -> x / sqrt(mean(x^2) + eps) * g."""
        r = 1.0 / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + float(np.float32(self.cfg.rms_eps)))
        return X * r * g

    def rope(self, Y: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """Rotate the pairs (i, i + hd/2) of every head of Y [T, heads * hd] at position pos[t]
        by the angle pos * theta^(-2i/hd)."""
        hd = self.cfg.head_dim
        half = hd // 2
        T = Y.shape[0]
        Yh = Y.reshape(T, -1, hd)
        i = np.arange(half, dtype=np.float64)
        ang = pos.astype(np.float64)[:, None] * float(np.float32(self.cfg.rope_theta)) ** (-2.0 * i / hd)
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        a, b = Yh[:, :, :half], Yh[:, :, half:]
        return np.concatenate([a * c - b * s, b * c + a * s], axis=2).reshape(T, -1)

    def attention(self, Q, Kall, Vall, pos0):
        """Causal softmax attention of the T query rows (positions pos0 + t) over the cached and new
        rows Kall, Vall [nkv][pos0 + T][hd]; query head h reads KV head h // (nq / nkv)."""
        cfg = self.cfg
        hd, nq, nkv = cfg.head_dim, cfg.n_heads, cfg.n_kv_heads
        G = nq // nkv
        T = Q.shape[0]
        n = pos0 + T
        mask = np.arange(n)[None, :] <= (pos0 + np.arange(T))[:, None]  # [T][n]
        O = np.empty((T, nq * hd))
        for h in range(nq):
            j = h // G
            S = Q[:, h * hd:(h + 1) * hd] @ Kall[j].T / np.sqrt(float(hd))
            S = np.where(mask, S, -np.inf)
            S -= S.max(axis=1, keepdims=True)
            E = np.exp(S)
            O[:, h * hd:(h + 1) * hd] = (E / E.sum(axis=1, keepdims=True)) @ Vall[j]
        return O

    def ffn(self, U: np.ndarray, l: int) -> np.ndarray:
        cfg = self.cfg
        if not getattr(cfg, "n_experts", 0):
            g = U @ self._mat("w_gate", l).T
            u = U @ self._mat("w_up", l).T
            return (g / (1.0 + np.exp(-g)) * u) @ self._mat("w_down", l).T
        # mixture of experts: softmax over all router logits, the A largest (ties to the lower
        # index), their probabilities renormalised, the weighted sum of the chosen SwiGLU experts
        E, A = cfg.n_experts, cfg.n_experts_active
        Z = U @ bf16_bits_to_f64(self.w["w_router"][l]).T  # [T][E]
        out = np.zeros_like(U)
        for t in range(U.shape[0]):
            z = Z[t]
            p = np.exp(z - z.max())
            p /= p.sum()
            order = np.lexsort((np.arange(E), -z))[:A]
            wts = p[order] / p[order].sum()
            for e, we in zip(order, wts):
                g = bf16_bits_to_f64(self.w["moe_gate"][l][e]) @ U[t]
                u = bf16_bits_to_f64(self.w["moe_up"][l][e]) @ U[t]
                out[t] += we * (bf16_bits_to_f64(self.w["moe_down"][l][e]) @ (g / (1.0 + np.exp(-g)) * u))
        return out

    def run(self, tokens, start_pos: int = 0, k_prefix=None, v_prefix=None):
        """Logits [T][V] of tokens at positions start_pos.., and the new K and V rows as bf16 bits
        [L][nkv][T][hd]. k_prefix, v_prefix: bf16 bits [L][nkv][>= start_pos][hd] (None when
        start_pos is 0)."""
        cfg = self.cfg
        toks = np.asarray(tokens, dtype=np.int64)
        T = len(toks)
        hd, nkv, L = cfg.head_dim, cfg.n_kv_heads, cfg.n_layers
        pos = start_pos + np.arange(T)
        X = bf16_bits_to_f64(np.asarray(self.w["embed"])[toks])
        knew = np.empty((L, nkv, T, hd), dtype=np.uint16)
        vnew = np.empty((L, nkv, T, hd), dtype=np.uint16)
        for l in range(L):
            U = self.rmsnorm(X, self._gain("attn_norm", l))
            Q = self.rope(U @ self._mat("wq", l).T, pos)
            K = round_to_bf16(self.rope(U @ self._mat("wk", l).T, pos)).reshape(T, nkv, hd).transpose(1, 0, 2)
            V = round_to_bf16(U @ self._mat("wv", l).T).reshape(T, nkv, hd).transpose(1, 0, 2)
            knew[l], vnew[l] = f64_to_bf16_bits(K), f64_to_bf16_bits(V)
            if start_pos > 0:
                Kall = np.concatenate([bf16_bits_to_f64(k_prefix[l][:, :start_pos]), K], axis=1)
                Vall = np.concatenate([bf16_bits_to_f64(v_prefix[l][:, :start_pos]), V], axis=1)
            else:
                Kall, Vall = K, V
            X = X + self.attention(Q, Kall, Vall, start_pos) @ self._mat("wo", l).T
            X = X + self.ffn(self.rmsnorm(X, self._gain("ffn_norm", l)), l)
        logits = self.rmsnorm(X, self._gain("final_norm")) @ self._mat("lm_head").T
        return logits, knew, vnew
