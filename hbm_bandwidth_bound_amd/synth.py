"""Seeded synthetic inputs: model shapes, weights, prompts.

This module generates *data* only. It holds none of the decoder's arithmetic, and it is the one
place both the CPU oracle's tests and the GPU path draw their inputs from.

Weights are "N(0, 0.02) bf16 from a seed". No generator is fixed by the shapes' description, so
the reading used here is a counter-based one that is bit-identical on the CPU (NumPy) and on the
GPU (torch integer ops), which lets the multi-GB configurations be generated on the device in
milliseconds while the oracle still sees exactly the same bits:

* each element's flat index ``i`` (row-major ``[out][in]``) is hashed with two tensor keys by the
  ``lowbias32`` integer mixer (C. Wellons' hash-prospector, 2020) into 64 random bits;
* the four 16-bit fields are summed (Irwin-Hall with n = 4: mean 131070, variance
  4·(65536²−1)/12), centred, and scaled in fp32 to standard deviation 0.02;
* the fp32 value is rounded to bf16 with round-to-nearest-even.

8-bit models (``weight_format`` 1) take the same bf16 values of every streamed matrix (the seven
per-layer matrices and the LM head) times 128, encoded as e4m3fn codes with round-to-nearest-even
by integer operations on the bit pattern (again identical on both backends), and give tensor t the
scale 2^-7 * (0.75 + 0.25 * (t mod 4)): a synthetic 8-bit checkpoint whose matrices differ in scale,
so that a scale applied to the wrong matrix shows. (The decoder itself never quantizes: it reads
the codes and scales it is given.) The embedding and the norm gains stay bf16.

RMSNorm gains are 1.0 (see ``norm_init``). Prompt ids are uniform in ``[0, V)`` by a
multiply-shift of a hashed counter.

The shapes are those of the decoder configurations: tiny (2 layers, d 256), the ~1.6B headline
model, the ~8B model, and the 128-expert mixture-of-experts model, plus two small
mixture-of-experts shapes and a two-layer cut of the full one for the parity tests.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

MASK32 = 0xFFFFFFFF


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab_size: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    n_experts: int = 0
    n_experts_active: int = 0
    expert_ffn_dim: int = 0
    weight_format: int = 0  # 0: bf16 matrices; 1: e4m3fn codes with one fp32 scale per matrix

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def scaled(self, **kw) -> "ModelConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named run: model, prompt length, decode steps, sampling."""
    name: str
    model: ModelConfig
    prompt_len: int
    decode_steps: int
    weight_seed: int = 0
    prompt_seed: int = 1
    sample_seed: int = 2
    top_k: int = 1
    temperature: float = 1.0

    @property
    def max_seq(self) -> int:
        return self.prompt_len + self.decode_steps


TINY = ModelConfig("tiny", 2, 256, 4, 2, 64, 1024, 4096)
M1_6B = ModelConfig("1.6b", 24, 2048, 16, 8, 128, 8192, 32768)
M8B = ModelConfig("8b", 32, 4096, 32, 8, 128, 14336, 128256)
MOE = ModelConfig("moe", 48, 2048, 32, 4, 128, 0, 151936, n_experts=128, n_experts_active=8,
                  expert_ffn_dim=768)

# Mixture-of-experts shapes for tests: 8 query heads on one KV head (the group of the full model),
# 1-tile expert rows (tiny) and 3-tile expert rows whose down-projection units span experts (small),
# and the full model's layer shape cut to two layers.
TINY_MOE = ModelConfig("tiny-moe", 2, 256, 8, 1, 128, 0, 4096, n_experts=16, n_experts_active=4,
                       expert_ffn_dim=256)
SMALL_MOE = ModelConfig("small-moe", 2, 512, 8, 1, 128, 0, 4096, n_experts=32, n_experts_active=8,
                        expert_ffn_dim=768)
MOE_2L = MOE.scaled(name="moe-2l", n_layers=2)

# 8-bit weights: the tile holds 512 weights of a row, so d_model, n_heads * head_dim and ffn_dim are
# multiples of 512 (the bf16 tiny shape is not): a small shape for the parity tests, and the 1.6B
# and 8B shapes with 8-bit matrices.
TINY_FP8 = ModelConfig("tiny-fp8", 2, 512, 8, 4, 64, 1536, 4096, weight_format=1)
M1_6B_FP8 = M1_6B.scaled(name="1.6b-fp8", weight_format=1)
M1_6B_FP8_2L = M1_6B.scaled(name="1.6b-fp8-2l", n_layers=2, weight_format=1)
M8B_FP8 = M8B.scaled(name="8b-fp8", weight_format=1)

# One GPU's share of the 1.6B model under 8-way tensor parallelism: QKV and gate/up split by
# output rows (2 query heads and their KV head, 1,024 of the FFN's 8,192), O and down by input
# columns (each GPU's partial residual update of all 2,048 outputs), the LM head by vocabulary
# (4,096 rows). On one GPU the all-reduce of the partial sums over a single member is the
# identity, so the share runs as a decoder of this shape; the 2-layer cut is a parity shape.
M1_6B_TP8 = M1_6B.scaled(name="1.6b-tp8", n_heads=2, n_kv_heads=1, ffn_dim=1024, vocab_size=4096)
M1_6B_TP8_2L = M1_6B_TP8.scaled(name="1.6b-tp8-2l", n_layers=2)

MODELS: Dict[str, ModelConfig] = {m.name: m for m in (TINY, M1_6B, M8B, MOE, TINY_MOE, SMALL_MOE, MOE_2L, TINY_FP8,
                                                       M1_6B_FP8, M1_6B_FP8_2L, M8B_FP8, M1_6B_TP8, M1_6B_TP8_2L)}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, 64, 32),
    "1.6b-1k": Workload("1.6b-1k", M1_6B, 1024, 512),
    "1.6b-1k-topk": Workload("1.6b-1k-topk", M1_6B, 1024, 512, top_k=50, temperature=0.8),
    "1.6b-32k": Workload("1.6b-32k", M1_6B, 32768, 256),
    "8b-2k": Workload("8b-2k", M8B, 2048, 256),
    "moe-1k": Workload("moe-1k", MOE, 1024, 256),
    "1.6b-1k-fp8": Workload("1.6b-1k-fp8", M1_6B_FP8, 1024, 512),
    "8b-2k-fp8": Workload("8b-2k-fp8", M8B_FP8, 2048, 256),
    "1.6b-tp8-1k": Workload("1.6b-tp8-1k", M1_6B_TP8, 1024, 512),
}

# Tensor numbering for the weight generator: 0 embed, 1 lm_head, then per layer l
# 2 + 7l + {0 wq, 1 wk, 2 wv, 3 wo, 4 w_gate, 5 w_up, 6 w_down}.
LAYER_MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


# Mixture-of-experts layers: the router [E][d] and the experts' matrices stacked per layer,
# gate and up [E][Fe][d], down [E][d][Fe]. The stacked matrices take the tensor numbers of w_gate,
# w_up and w_down; the router of layer l is tensor ROUTER_TENSOR + l.
MOE_MATS = ("w_router", "moe_gate", "moe_up", "moe_down")
ROUTER_TENSOR = 0x40000000


def layer_mats(cfg: ModelConfig):
    if cfg.n_experts:
        return ("wq", "wk", "wv", "wo") + MOE_MATS
    return LAYER_MATS


def mat_shape(cfg: ModelConfig, name: str):
    d, q, kv, f = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.ffn_dim
    E, Fe = cfg.n_experts, cfg.expert_ffn_dim
    return {"wq": (q, d), "wk": (kv, d), "wv": (kv, d), "wo": (d, q), "w_gate": (f, d),
            "w_up": (f, d), "w_down": (d, f), "embed": (cfg.vocab_size, d),
            "lm_head": (cfg.vocab_size, d), "w_router": (E, d), "moe_gate": (E, Fe, d),
            "moe_up": (E, Fe, d), "moe_down": (E, d, Fe)}[name]


def tensor_index(name: str, layer: Optional[int] = None) -> int:
    if name == "embed":
        return 0
    if name == "lm_head":
        return 1
    if name == "w_router":
        return ROUTER_TENSOR + layer
    alias = {"moe_gate": "w_gate", "moe_up": "w_up", "moe_down": "w_down"}
    return 2 + 7 * layer + LAYER_MATS.index(alias.get(name, name))


# ----------------------------------------------------------------------------------------------
# Counter-based generator (NumPy or torch backend; integer ops only until one fp32 multiply)
# ----------------------------------------------------------------------------------------------

def _lowbias32_scalar(x: int) -> int:
    x &= MASK32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & MASK32
    x ^= x >> 15
    x = (x * 0x846CA68B) & MASK32
    x ^= x >> 16
    return x


def tensor_keys(seed: int, tidx: int):
    a = _lowbias32_scalar(seed * 0x9E3779B9 + 0x632BE5AB)
    k1 = _lowbias32_scalar(a ^ _lowbias32_scalar(tidx * 2 + 1))
    k2 = _lowbias32_scalar(a ^ _lowbias32_scalar(tidx * 2 + 2) ^ 0x5BD1E995)
    return k1, k2


def _mul32(xp, x, c: int):
    """(x * c) mod 2^32 for x < 2^32 held in int64, without int64 overflow."""
    lo = c & 0xFFFF
    hi = c >> 16
    return ((((x * hi) & 0xFFFF) << 16) + x * lo) & MASK32


def _mix32(xp, x):
    x = x ^ (x >> 16)
    x = _mul32(xp, x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(xp, x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


# sigma of the centred Irwin-Hall(4) sum of 16-bit uniforms
_IH_SIGMA = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
WEIGHT_STD = 0.02
_IH_SCALE_F32 = np.float32(WEIGHT_STD / _IH_SIGMA)


def _bf16_rne_bits_from_f32_bits(xp, u):
    """fp32 bit pattern (int64 holding uint32) -> bf16 bits with round-to-nearest-even."""
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r & 0xFFFF


def _mix32_u32(x: np.ndarray) -> np.ndarray:
    """lowbias32 on a uint32 array (NumPy multiplies wrap modulo 2^32)."""
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(0x7FEB352D)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(0x846CA68B)
    x = x ^ (x >> np.uint32(16))
    return x


def _weights_bits_np(shape, seed: int, tidx: int, std: float = WEIGHT_STD) -> np.ndarray:
    k1, k2 = tensor_keys(seed, tidx)
    scale = np.float32(std / _IH_SIGMA)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 22
    m16 = np.uint32(0xFFFF)
    for s in range(0, n, chunk):
        i = np.arange(s, min(n, s + chunk), dtype=np.uint32)
        h1 = _mix32_u32(i ^ np.uint32(k1))
        h2 = _mix32_u32(i ^ np.uint32(k2))
        t = ((h1 & m16) + (h1 >> np.uint32(16)) + (h2 & m16) + (h2 >> np.uint32(16))).astype(np.int32) - 131070
        x = t.astype(np.float32) * scale
        u = x.view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[s:s + len(i)] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(shape)


def _weights_bits_torch(shape, seed: int, tidx: int, device, std: float = WEIGHT_STD):
    import torch
    k1, k2 = tensor_keys(seed, tidx)
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.int16, device=device)
    chunk = 1 << 26
    scale = torch.tensor(float(np.float32(std / _IH_SIGMA)), dtype=torch.float32, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        i = torch.arange(s, e, dtype=torch.int64, device=device)
        h1 = _mix32(torch, i ^ k1)
        h2 = _mix32(torch, i ^ k2)
        t = ((h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16)) - 131070
        x = t.to(torch.float32) * scale
        u = x.view(torch.int32).to(torch.int64) & MASK32
        b = _bf16_rne_bits_from_f32_bits(torch, u)
        out[s:e] = (b - ((b >> 15) << 16)).to(torch.int16)  # store the 16 bits as int16
    return out.view(shape)


FP8_MATS = LAYER_MATS + ("lm_head",)


def fp8_scale(tidx: int) -> float:
    """Scale of tensor tidx of an 8-bit model (exact in fp32)."""
    return 2.0 ** -7 * (0.75 + 0.25 * (tidx % 4))


def fp8_scales(cfg: ModelConfig) -> np.ndarray:
    """[n_layers * 7 + 1] fp32: per layer wq, wk, wv, wo, w_gate, w_up, w_down, then lm_head."""
    sc = [fp8_scale(tensor_index(m, l)) for l in range(cfg.n_layers) for m in LAYER_MATS]
    return np.array(sc + [fp8_scale(tensor_index("lm_head"))], dtype=np.float32)


def _e4m3_codes(xp, b):
    """bf16 bit patterns (int64) -> e4m3fn codes of 128 times their values, round to nearest even.

    Integer operations on the fp32 pattern (b << 16, exponent raised by 7): exponents >= 121 give
    normal codes (3 mantissa bits kept, a carry may raise the exponent), smaller ones the subnormal
    codes m * 2^-9 (m = 0..8; 8 is the smallest normal code). The inputs here stay far below 448.
    """
    u = (b & 0xFFFF) << 16
    sign = (u >> 31) & 1
    a = u & 0x7FFFFFFF
    a = xp.where(a == 0, a, a + (7 << 23))
    e = a >> 23
    mant = a & 0x7FFFFF
    m3 = mant >> 20
    rem = mant & 0xFFFFF
    up = ((rem > 0x80000) | ((rem == 0x80000) & ((m3 & 1) == 1))).astype(m3.dtype) if xp is np else \
        ((rem > 0x80000) | ((rem == 0x80000) & ((m3 & 1) == 1))).to(m3.dtype)
    normal = (((e - 120) << 3) | m3) + up
    sig = mant | 0x800000
    shift = xp.clip(141 - e, 21, 40) if xp is np else (141 - e).clamp(21, 40)
    q = sig >> shift
    r = sig - (q << shift)
    half = xp.ones_like(r) << (shift - 1)
    upq = (r > half) | ((r == half) & ((q & 1) == 1))
    sub = q + (upq.astype(q.dtype) if xp is np else upq.to(q.dtype))
    sub = xp.where(e == 0, xp.zeros_like(sub), sub)
    code = xp.where(e >= 121, normal, sub)
    code = xp.minimum(code, xp.full_like(code, 0x7E))
    return code | (sign << 7)


def fp8_codes_np(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> uint8 e4m3fn codes (see _e4m3_codes)."""
    return _e4m3_codes(np, bits.astype(np.int64)).astype(np.uint8)


def fp8_codes_torch(bits):
    """int16 bf16 bits (torch) -> uint8 codes on the same device, chunked."""
    import torch
    flat = bits.reshape(-1)
    out = torch.empty(flat.numel(), dtype=torch.uint8, device=flat.device)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        b = flat[s:s + chunk].to(torch.int64) & 0xFFFF
        out[s:s + chunk] = _e4m3_codes(torch, b).to(torch.uint8)
    return out.view(bits.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def norm_init(cfg: ModelConfig, mode: str = "ones") -> np.ndarray:
    """RMSNorm gains. 'ones' (the default reading) gives 1.0 = 0x3F80 in bf16."""
    if mode != "ones":
        raise ValueError("only 'ones' norm gains are generated")
    return np.full(cfg.d_model, 0x3F80, dtype=np.uint16)


def make_weights_np(cfg: ModelConfig, seed: int = 0) -> Dict[str, object]:
    """All weights as bf16 bit arrays (uint16), keyed like the C-ABI weight struct."""
    w: Dict[str, object] = {
        "embed": _weights_bits_np(mat_shape(cfg, "embed"), seed, 0),
        "lm_head": _weights_bits_np(mat_shape(cfg, "lm_head"), seed, 1),
        "final_norm": norm_init(cfg),
    }
    for name in ("attn_norm", "ffn_norm"):
        w[name] = [norm_init(cfg) for _ in range(cfg.n_layers)]
    for name in layer_mats(cfg):
        w[name] = [_weights_bits_np(mat_shape(cfg, name), seed, tensor_index(name, l))
                   for l in range(cfg.n_layers)]
    if cfg.weight_format == 1:
        for name in FP8_MATS:
            w[name] = [fp8_codes_np(a) for a in w[name]] if isinstance(w[name], list) else fp8_codes_np(w[name])
        w["w_scale"] = fp8_scales(cfg)
    return w


def make_weights_torch(cfg: ModelConfig, seed: int = 0, device="cuda") -> Dict[str, object]:
    """Same bits as make_weights_np, produced on a torch device (int16 tensors)."""
    import torch
    w: Dict[str, object] = {
        "embed": _weights_bits_torch(mat_shape(cfg, "embed"), seed, 0, device),
        "lm_head": _weights_bits_torch(mat_shape(cfg, "lm_head"), seed, 1, device),
        "final_norm": torch.full((cfg.d_model,), 0x3F80, dtype=torch.int16, device=device),
    }
    for name in ("attn_norm", "ffn_norm"):
        w[name] = [torch.full((cfg.d_model,), 0x3F80, dtype=torch.int16, device=device)
                   for _ in range(cfg.n_layers)]
    for name in layer_mats(cfg):
        w[name] = [_weights_bits_torch(mat_shape(cfg, name), seed, tensor_index(name, l), device)
                   for l in range(cfg.n_layers)]
    if cfg.weight_format == 1:
        for name in FP8_MATS:
            w[name] = [fp8_codes_torch(t) for t in w[name]] if isinstance(w[name], list) else fp8_codes_torch(w[name])
        w["w_scale"] = fp8_scales(cfg)
    return w


def weights_torch_to_np(w) -> Dict[str, object]:
    """Copy a torch weight dict to host uint16 arrays (the oracle's input format)."""
    def cv(t):
        a = t.cpu().numpy()
        return a if a.dtype == np.uint8 else a.view(np.uint16)
    out = {}
    for k, v in w.items():
        if isinstance(v, np.ndarray):
            out[k] = v
            continue
        out[k] = [cv(t) for t in v] if isinstance(v, list) else cv(v)
    return out


def prompt_ids(n: int, vocab: int, seed: int = 1) -> np.ndarray:
    """n uniform token ids in [0, vocab)."""
    k1, _ = tensor_keys(seed, 0x7FFF0000)
    i = np.arange(n, dtype=np.int64)
    h = _mix32(np, i ^ k1)
    return ((h * vocab) >> 32).astype(np.int32)


# Synthetic KV-cache contents: K and V rows of positions 0..n-1 as bf16 bits, [L][nkv][n][hd]
# each, drawn like the weights but with standard deviation `std` (so that attention weights are
# far from uniform). Used where a context longer than the oracle can prefill is needed: both
# sides start from the same rows.
KV_TENSOR_K = 0x7FFE0000
KV_TENSOR_V = 0x7FFE0001


def kv_shape(cfg: ModelConfig, n: int):
    return (cfg.n_layers, cfg.n_kv_heads, n, cfg.head_dim)


def synthetic_kv_np(cfg: ModelConfig, n: int, seed: int = 7, std: float = 1.0):
    return (_weights_bits_np(kv_shape(cfg, n), seed, KV_TENSOR_K, std),
            _weights_bits_np(kv_shape(cfg, n), seed, KV_TENSOR_V, std))


def synthetic_kv_torch(cfg: ModelConfig, n: int, seed: int = 7, device="cuda", std: float = 1.0):
    """Same bits as synthetic_kv_np, as int16 tensors on a torch device."""
    return (_weights_bits_torch(kv_shape(cfg, n), seed, KV_TENSOR_K, device, std),
            _weights_bits_torch(kv_shape(cfg, n), seed, KV_TENSOR_V, device, std))
