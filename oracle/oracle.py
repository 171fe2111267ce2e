"""ctypes front end of ``oracle.c`` (test infrastructure only).

Arrays go in as NumPy arrays (bf16 as uint16 bit patterns). Nothing here computes part of the
decoder: every arithmetic step runs in the C file.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP for row splitting only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = C.CDLL(_LIB)
        f32p = C.POINTER(C.c_float)
        f64p = C.POINTER(C.c_double)
        u16p = C.POINTER(C.c_uint16)
        i32p = C.POINTER(C.c_int32)
        lib.oc_gemv.argtypes = [u16p, f32p, f32p, C.c_int, C.c_int]
        lib.oc_rmsnorm.argtypes = [f32p, u16p, f32p, C.c_int, C.c_float]
        lib.oc_rope.argtypes = [f32p, C.c_int, C.c_int, C.c_float]
        lib.oc_silu.argtypes = [C.c_float]
        lib.oc_silu.restype = C.c_float
        lib.oc_attend.argtypes = [f32p, u16p, u16p, C.c_int, C.c_int, C.c_size_t, f32p, f64p]
        lib.oc_argmax.argtypes = [f32p, C.c_int]
        lib.oc_argmax.restype = C.c_int
        lib.oc_topk_sample.argtypes = [f32p, C.c_int, C.c_int, C.c_float, C.c_uint64, C.c_int64, i32p, f64p,
                                       f64p]
        lib.oc_topk_sample.restype = C.c_int
        lib.oc_splitmix64.argtypes = [C.c_uint64]
        lib.oc_splitmix64.restype = C.c_uint64
        lib.oc_uniform.argtypes = [C.c_uint64, C.c_int64]
        lib.oc_uniform.restype = C.c_double
        lib.oc_f32_to_bf16.argtypes = [C.c_float]
        lib.oc_f32_to_bf16.restype = C.c_uint16
        lib.oc_bf16_to_f32.argtypes = [C.c_uint16]
        lib.oc_bf16_to_f32.restype = C.c_float
        lib.oc_set_threads.argtypes = [C.c_int]
        lib.oc_set_gemv_order.argtypes = [C.c_int]
        lib.oc_step.argtypes = [C.c_void_p, C.c_void_p, u16p, u16p, C.c_int, C.c_int, f32p]
        lib.oc_step.restype = C.c_int
        lib.oc_full_recompute.argtypes = [C.c_void_p, C.c_void_p, i32p, C.c_int, f32p]
        lib.oc_full_recompute.restype = C.c_int
        lib.oc_moe_route.argtypes = [f32p, C.c_int, C.c_int, i32p, f64p]
        lib.oc_moe_route.restype = C.c_int
        lib.oc_moe_ffn.argtypes = [C.c_void_p, C.c_void_p, C.c_int, f32p, f32p, f32p]
        lib.oc_moe_ffn.restype = None
        lib.oc_set_route_log.argtypes = [f32p, C.c_int]
        lib.oc_set_route_log.restype = None
        u8p = C.POINTER(C.c_uint8)
        lib.oc_e4m3_to_f32.argtypes = [C.c_uint8]
        lib.oc_e4m3_to_f32.restype = C.c_float
        lib.oc_gemv_e4m3.argtypes = [u8p, C.c_float, f32p, f32p, C.c_int, C.c_int]
        lib.oc_gemv_e4m3.restype = None
        _lib = lib
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(C.POINTER(ct))


def set_threads(n: int) -> None:
    _load().oc_set_threads(int(n))


def set_gemv_order(descending: bool) -> None:
    """Sum every GEMV row in descending instead of ascending k order (a second valid rounding of
    the same model; used only to measure the model's own sensitivity to rounding order)."""
    _load().oc_set_gemv_order(1 if descending else 0)


def gemv(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float32)
    _load().oc_gemv(_p(W, C.c_uint16), _p(x, C.c_float), _p(y, C.c_float), rows, cols)
    return y


def e4m3_to_f32(code: int) -> float:
    """Value of one fp8 e4m3fn code (0..255)."""
    return float(_load().oc_e4m3_to_f32(int(code) & 0xFF))


def gemv_e4m3(W: np.ndarray, scale: float, x: np.ndarray) -> np.ndarray:
    """scale * (decoded W) x for a [rows][cols] matrix of e4m3fn codes (uint8)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float32)
    _load().oc_gemv_e4m3(_p(W, C.c_uint8), float(scale), _p(x, C.c_float), _p(y, C.c_float), rows, cols)
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.uint16)
    u = np.empty_like(x)
    _load().oc_rmsnorm(_p(x, C.c_float), _p(g, C.c_uint16), _p(u, C.c_float), len(x), eps)
    return u


def rope(y: np.ndarray, pos: int, theta: float) -> np.ndarray:
    y = np.array(y, dtype=np.float32, copy=True)
    _load().oc_rope(_p(y, C.c_float), len(y), int(pos), theta)
    return y


def silu(g: float) -> float:
    return float(_load().oc_silu(float(g)))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Softmax attention of q [hd] over K, V [n][hd] (bf16 bits). Returns (out [hd], probs [n])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    n, hd = K.shape
    out = np.empty(hd, dtype=np.float32)
    probs = np.empty(max(n, 1), dtype=np.float64)
    _load().oc_attend(_p(q, C.c_float), _p(K, C.c_uint16), _p(V, C.c_uint16), n, hd, hd, _p(out, C.c_float),
                      _p(probs, C.c_double))
    return out, probs[:n]


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return int(_load().oc_argmax(_p(v, C.c_float), len(v)))


def topk_sample(logits: np.ndarray, k: int, temperature: float, seed: int, pos: int):
    """Returns (token, candidate ids [k], candidate probabilities [k], u)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    kk = max(1, min(k, len(logits)))
    idx = np.empty(kk, dtype=np.int32)
    p = np.empty(kk, dtype=np.float64)
    u = C.c_double(0.0)
    tok = _load().oc_topk_sample(_p(logits, C.c_float), len(logits), k, temperature, seed & (2**64 - 1), pos,
                                 _p(idx, C.c_int32), _p(p, C.c_double), C.byref(u))
    return int(tok), idx, p, float(u.value)


def moe_route(z: np.ndarray, active: int):
    """Router of a mixture-of-experts layer: (expert ids [A] in rank order, weights [A] fp64)."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    idx = np.empty(active, dtype=np.int32)
    w = np.empty(active, dtype=np.float64)
    if _load().oc_moe_route(_p(z, C.c_float), len(z), int(active), _p(idx, C.c_int32), _p(w, C.c_double)) != 0:
        raise ValueError("bad router sizes")
    return idx, w


def splitmix64(x: int) -> int:
    return int(_load().oc_splitmix64(x & (2**64 - 1)))


def uniform(seed: int, pos: int) -> float:
    return float(_load().oc_uniform(seed & (2**64 - 1), pos))


def f32_to_bf16(x: float) -> int:
    return int(_load().oc_f32_to_bf16(float(x)))


def bf16_to_f32(b: int) -> float:
    return float(_load().oc_bf16_to_f32(int(b)))


class _Cfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab_size", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("max_seq", C.c_int32), ("n_experts", C.c_int32), ("n_experts_active", C.c_int32),
                ("expert_ffn_dim", C.c_int32), ("weight_format", C.c_int32)]


_PP = C.POINTER(C.POINTER(C.c_uint16))


class _W(C.Structure):
    _fields_ = [("embed", C.POINTER(C.c_uint16)), ("final_norm", C.POINTER(C.c_uint16)),
                ("lm_head", C.POINTER(C.c_uint16)), ("attn_norm", _PP), ("wq", _PP), ("wk", _PP),
                ("wv", _PP), ("wo", _PP), ("ffn_norm", _PP), ("w_gate", _PP), ("w_up", _PP),
                ("w_down", _PP), ("w_router", _PP), ("moe_gate", _PP), ("moe_up", _PP), ("moe_down", _PP),
                ("w_scale", C.POINTER(C.c_float))]


_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
_MOE_KEYS = ("w_router", "moe_gate", "moe_up", "moe_down")


class OracleModel:
    """The decoder of one configuration with its own bf16 KV cache.

    ``cfg`` needs attributes n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size,
    rms_eps, rope_theta, n_experts, n_experts_active, expert_ffn_dim. ``weights`` maps names to
    uint16 arrays (per-layer names to lists). A mixture-of-experts model (n_experts > 0) has
    w_router, moe_gate, moe_up, moe_down per layer instead of w_gate, w_up, w_down. With
    ``cfg.weight_format == 1`` (optional attribute, default 0) wq, wk, wv, wo, w_gate, w_up, w_down
    and lm_head are uint8 arrays of e4m3fn codes and ``weights["w_scale"]`` holds the fp32 scales
    [n_layers * 7 + 1] (per layer wq, wk, wv, wo, w_gate, w_up, w_down; then lm_head).
    """

    def __init__(self, cfg, weights: Dict[str, object], max_seq: int):
        self.cfg = cfg
        self.max_seq = int(max_seq)
        self._keep = []
        self._c = _Cfg(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
                       cfg.vocab_size, cfg.rms_eps, cfg.rope_theta, self.max_seq, cfg.n_experts,
                       cfg.n_experts_active, cfg.expert_ffn_dim, int(getattr(cfg, "weight_format", 0)))

        def arr(a):  # bf16 bit patterns, or bytes (fp8 codes) passed through the same pointer type
            a = np.asarray(a)
            a = np.ascontiguousarray(a, dtype=np.uint8 if a.dtype == np.uint8 else np.uint16)
            self._keep.append(a)
            return a.ctypes.data_as(C.POINTER(C.c_uint16))

        def arrs(lst):
            ptrs = (C.POINTER(C.c_uint16) * len(lst))(*[arr(a) for a in lst])
            self._keep.append(ptrs)
            return C.cast(ptrs, _PP)

        def arrs_opt(k):
            return arrs(weights[k]) if k in weights else C.cast(None, _PP)

        if "w_scale" in weights:
            sc = np.ascontiguousarray(weights["w_scale"], dtype=np.float32)
            self._keep.append(sc)
            scp = sc.ctypes.data_as(C.POINTER(C.c_float))
        else:
            scp = C.cast(None, C.POINTER(C.c_float))
        self._w = _W(arr(weights["embed"]), arr(weights["final_norm"]), arr(weights["lm_head"]),
                     *[arrs_opt(k) for k in _LAYER_KEYS + _MOE_KEYS], scp)
        kv_elems = cfg.n_layers * cfg.n_kv_heads * self.max_seq * cfg.head_dim
        self.kcache = np.zeros(kv_elems, dtype=np.uint16)
        self.vcache = np.zeros(kv_elems, dtype=np.uint16)
        self.pos = 0

    def kv_view(self):
        shape = (self.cfg.n_layers, self.cfg.n_kv_heads, self.max_seq, self.cfg.head_dim)
        return self.kcache.reshape(shape), self.vcache.reshape(shape)

    def step(self, token: int, pos: Optional[int] = None) -> np.ndarray:
        pos = self.pos if pos is None else int(pos)
        logits = np.empty(self.cfg.vocab_size, dtype=np.float32)
        rc = _load().oc_step(C.byref(self._c), C.byref(self._w), _p(self.kcache, C.c_uint16),
                             _p(self.vcache, C.c_uint16), int(token), pos, _p(logits, C.c_float))
        if rc != 0:
            raise ValueError(f"oracle step rejected token={token} pos={pos}")
        self.pos = pos + 1
        return logits

    def run(self, tokens: Sequence[int], start_pos: int = 0) -> np.ndarray:
        """Feed tokens at positions start_pos.. and return all their logits [n][V]."""
        out = np.empty((len(tokens), self.cfg.vocab_size), dtype=np.float32)
        for i, t in enumerate(tokens):
            out[i] = self.step(int(t), start_pos + i)
        return out

    def full_recompute(self, tokens: Sequence[int]) -> np.ndarray:
        return full_recompute(self, tokens)

    def moe_ffn(self, layer: int, u: np.ndarray):
        """Feed-forward output of mixture-of-experts layer `layer` for the normalised input u [d]:
        (y [d], router logits [E])."""
        u = np.ascontiguousarray(u, dtype=np.float32)
        y = np.empty(self.cfg.d_model, dtype=np.float32)
        z = np.empty(self.cfg.n_experts, dtype=np.float32)
        _load().oc_moe_ffn(C.byref(self._c), C.byref(self._w), int(layer), _p(u, C.c_float), _p(y, C.c_float),
                           _p(z, C.c_float))
        return y, z

    def record_routes(self, max_pos: int):
        """Start recording the router logits of step() at positions < max_pos; returns the
        [max_pos][n_layers][n_experts] fp32 array that fills in."""
        buf = np.full((max_pos, self.cfg.n_layers, self.cfg.n_experts), np.nan, dtype=np.float32)
        self._route_buf = buf
        _load().oc_set_route_log(_p(buf, C.c_float), int(max_pos))
        return buf

    def stop_recording(self):
        _load().oc_set_route_log(C.cast(None, C.POINTER(C.c_float)), 0)
        self._route_buf = None


def full_recompute(model: OracleModel, tokens: Sequence[int]) -> np.ndarray:
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    n = len(toks)
    out = np.empty((n, model.cfg.vocab_size), dtype=np.float32)
    rc = _load().oc_full_recompute(C.byref(model._c), C.byref(model._w), _p(toks, C.c_int32), n,
                                   _p(out, C.c_float))
    if rc != 0:
        raise ValueError("oracle full recompute rejected its input")
    return out
