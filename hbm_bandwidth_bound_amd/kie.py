"""ctypes binding of libkie.so (include/kie.h, include/kie_measure.h).

Argument marshalling only: torch is used for device memory and the stream; every step of the
decoder runs in the library's HIP kernels. Importing this module does not touch the GPU. Loading
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkie.so")

KIE_OK = 0
STATUS = {0: "KIE_OK", -1: "KIE_ERR_INVALID_ARG", -2: "KIE_ERR_UNSUPPORTED", -3: "KIE_ERR_CAPACITY",
          -4: "KIE_ERR_HIP", -5: "KIE_ERR_STATE", -6: "KIE_ERR_TIMEOUT", -7: "KIE_ERR_ABORTED"}


class KieError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class kie_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_dim", C.c_int32),
                ("vocab_size", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("max_seq_len", C.c_int32), ("n_experts", C.c_int32), ("n_experts_active", C.c_int32),
                ("expert_ffn_dim", C.c_int32), ("weight_format", C.c_int32)]


_U16P = C.POINTER(C.c_uint16)
_U16PP = C.POINTER(_U16P)


class kie_weights(C.Structure):
    _fields_ = [("embed", _U16P), ("final_norm", _U16P), ("lm_head", _U16P), ("attn_norm", _U16PP),
                ("wq", _U16PP), ("wk", _U16PP), ("wv", _U16PP), ("wo", _U16PP), ("ffn_norm", _U16PP),
                ("w_gate", _U16PP), ("w_up", _U16PP), ("w_down", _U16PP), ("w_router", _U16PP),
                ("moe_gate", _U16PP), ("moe_up", _U16PP), ("moe_down", _U16PP),
                ("weight_scales", C.POINTER(C.c_float))]

_LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down", "w_router", "moe_gate",
               "moe_up", "moe_down")


class kie_sampling(C.Structure):
    _fields_ = [("top_k", C.c_int32), ("temperature", C.c_float), ("seed", C.c_uint64)]


_lib = None


def load() -> C.CDLL:
    """Load libkie.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hbm_bandwidth_bound_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp = C.c_void_p
    i32p = C.POINTER(C.c_int32)
    cfgp = C.POINTER(kie_config)
    lib.kie_packed_weight_bytes.argtypes = [cfgp]
    lib.kie_packed_weight_bytes.restype = C.c_size_t
    lib.kie_kv_cache_bytes.argtypes = [cfgp]
    lib.kie_kv_cache_bytes.restype = C.c_size_t
    lib.kie_workspace_bytes.argtypes = [cfgp]
    lib.kie_workspace_bytes.restype = C.c_size_t
    lib.kie_create.argtypes = [cfgp, C.POINTER(kie_weights), vp, vp, vp, vp, C.POINTER(vp)]
    lib.kie_create.restype = C.c_int32
    lib.kie_create_static.argtypes = [cfgp, C.POINTER(kie_weights), vp, vp, vp, C.POINTER(vp)]
    lib.kie_create_static.restype = C.c_int32
    lib.kie_prefill.argtypes = [vp, vp, C.c_int32, vp, vp, C.POINTER(kie_sampling)]
    lib.kie_prefill.restype = C.c_int32
    lib.kie_decode_step.argtypes = [vp, vp, C.POINTER(kie_sampling), vp, vp]
    lib.kie_decode_step.restype = C.c_int32
    lib.kie_generate.argtypes = [vp, vp, C.c_int32, C.POINTER(kie_sampling), vp, vp, vp]
    lib.kie_generate.restype = C.c_int32
    lib.kie_sync.argtypes = [vp]
    lib.kie_sync.restype = C.c_int32
    lib.kie_reset.argtypes = [vp]
    lib.kie_reset.restype = C.c_int32
    lib.kie_set_token_stream.argtypes = [vp, vp, C.c_int32]
    lib.kie_set_token_stream.restype = C.c_int32
    lib.kie_set_skew.argtypes = [vp, C.c_uint32]
    lib.kie_set_skew.restype = C.c_int32
    lib.kie_set_abort_flag.argtypes = [vp, vp]
    lib.kie_set_abort_flag.restype = C.c_int32
    lib.kie_set_wait_timeout.argtypes = [vp, C.c_uint64]
    lib.kie_set_wait_timeout.restype = C.c_int32
    lib.kie_set_position.argtypes = [vp, C.c_int32]
    lib.kie_set_position.restype = C.c_int32
    lib.kie_position.argtypes = [vp]
    lib.kie_position.restype = C.c_int32
    lib.kie_status_string.argtypes = [C.c_int32]
    lib.kie_status_string.restype = C.c_char_p
    lib.kie_last_error.argtypes = [vp]
    lib.kie_last_error.restype = C.c_char_p
    lib.kie_destroy.argtypes = [vp]
    lib.kie_destroy.restype = None
    lib.kie_num_workgroups.argtypes = []
    lib.kie_num_workgroups.restype = C.c_int32
    lib.kie_stream_copy.argtypes = [vp, vp, C.c_size_t, vp]
    lib.kie_stream_copy.restype = C.c_int32
    lib.kie_stream_read.argtypes = [vp, C.c_size_t, vp, vp]
    lib.kie_stream_read.restype = C.c_int32
    lib.kie_probe_pingpong.argtypes = [C.c_int32, C.c_int32, C.c_int32, vp, vp, vp]
    lib.kie_probe_pingpong.restype = C.c_int32
    lib.kie_probe_allgather.argtypes = [C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, vp, vp]
    lib.kie_probe_allgather.restype = C.c_int32
    lib.kie_probe_page_latency.argtypes = [C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, vp, vp]
    lib.kie_probe_page_latency.restype = C.c_int32
    _lib = lib
    return lib


def make_config(model, max_seq: int) -> kie_config:
    return kie_config(model.n_layers, model.d_model, model.n_heads, model.n_kv_heads, model.head_dim,
                      model.ffn_dim, model.vocab_size, model.rms_eps, model.rope_theta, int(max_seq),
                      model.n_experts, model.n_experts_active, model.expert_ffn_dim,
                      int(getattr(model, "weight_format", 0)))


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(None)


def _check(lib, status: int, ctx=None):
    if status != KIE_OK:
        msg = lib.kie_last_error(ctx).decode(errors="replace")
        raise KieError(status, msg)


def sampling(top_k: int = 1, temperature: float = 1.0, seed: int = 0) -> kie_sampling:
    return kie_sampling(int(top_k), float(temperature), int(seed) & (2 ** 64 - 1))


class Engine:
    """A decode context over torch-owned device buffers.

    weights: dict of torch int16/uint16-bit tensors on the device (keys as in kie_weights; per-layer
    keys hold lists; a dense model has no w_router/moe_* keys, a mixture-of-experts model no
    w_gate/w_up/w_down). An 8-bit model (``model.weight_format == 1``) has uint8 code tensors for
    wq, wk, wv, wo, w_gate, w_up, w_down and lm_head, and ``weights["w_scale"]``: the
    n_layers * 7 + 1 fp32 matrix scales as a host array. The packed image, KV cache and workspace are allocated here as torch
    tensors (no workspace with ``static_workspace=True``: kie_create_static).
    """

    def __init__(self, model, weights: Dict[str, object], max_seq: int, stream=None, static_workspace=False):
        import torch
        self.torch = torch
        self.lib = load()
        self.model = model
        self.cfg = make_config(model, max_seq)
        lib = self.lib
        dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        nb_packed = lib.kie_packed_weight_bytes(C.byref(self.cfg))
        nb_kv = lib.kie_kv_cache_bytes(C.byref(self.cfg))
        nb_ws = lib.kie_workspace_bytes(C.byref(self.cfg))
        if not (nb_packed and nb_kv and nb_ws):
            raise KieError(-2, "configuration rejected by the library: " + lib.kie_last_error(None).decode())
        self.packed = torch.empty(nb_packed, dtype=torch.uint8, device=dev)
        self.kv = torch.empty(nb_kv // 2, dtype=torch.int16, device=dev)
        # static_workspace: kie_create_static, whose workspace is the library's own per-GPU array
        self.workspace = None if static_workspace else torch.empty(nb_ws, dtype=torch.uint8, device=dev)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        L = model.n_layers

        def p(t):
            return C.cast(C.c_void_p(t.data_ptr()), _U16P)

        def arr(lst):
            a = (_U16P * L)(*[p(t) for t in lst])
            return C.cast(a, _U16PP), a

        keep = []
        fields = {}
        for k in _LAYER_KEYS:
            if k in weights:
                ptrs, a = arr(weights[k])
                keep.append(a)
                fields[k] = ptrs
            else:
                fields[k] = C.cast(None, _U16PP)
        if "w_scale" in weights:
            import numpy as np
            sc = np.ascontiguousarray(weights["w_scale"], dtype=np.float32)
            keep.append(sc)
            scp = sc.ctypes.data_as(C.POINTER(C.c_float))
        else:
            scp = C.cast(None, C.POINTER(C.c_float))
        self._w = kie_weights(p(weights["embed"]), p(weights["final_norm"]), p(weights["lm_head"]),
                              *[fields[k] for k in _LAYER_KEYS], scp)
        self._keep = keep
        ctx = C.c_void_p()
        if static_workspace:
            st = lib.kie_create_static(C.byref(self.cfg), C.byref(self._w), _ptr(self.packed), _ptr(self.kv),
                                       C.c_void_p(self.stream.cuda_stream), C.byref(ctx))
        else:
            st = lib.kie_create(C.byref(self.cfg), C.byref(self._w), _ptr(self.packed), _ptr(self.kv),
                                _ptr(self.workspace), C.c_void_p(self.stream.cuda_stream), C.byref(ctx))
        _check(lib, st, None)
        self.ctx = ctx
        # the packing reads the source weights: keep them until the first sync
        self._src = weights
        self.sync()
        self._src = None
        self._tok = torch.zeros(1, dtype=torch.int32, device=dev)

    # ---------------------------------------------------------------- calls
    def sync(self):
        _check(self.lib, self.lib.kie_sync(self.ctx), self.ctx)

    def reset(self):
        _check(self.lib, self.lib.kie_reset(self.ctx), self.ctx)

    def set_position(self, pos: int):
        _check(self.lib, self.lib.kie_set_position(self.ctx, int(pos)), self.ctx)

    def set_skew(self, level: int):
        """Protocol stress (tests): workgroups idle pseudo-random amounts before stage boundaries."""
        _check(self.lib, self.lib.kie_set_skew(self.ctx, int(level)), self.ctx)

    def set_abort_flag(self, word=None):
        """word: pinned host int32 tensor of one element that the device reads (None removes it)."""
        st = self.lib.kie_set_abort_flag(self.ctx, _ptr(word) if word is not None else None)
        _check(self.lib, st, self.ctx)
        self._abort_word = word  # kept alive while installed

    def set_wait_timeout(self, microseconds: int):
        """Time limit of every device-side wait of later launches (0: the default)."""
        _check(self.lib, self.lib.kie_set_wait_timeout(self.ctx, int(microseconds)), self.ctx)

    def set_token_stream(self, ring=None):
        """ring: pinned host int32 tensor of 1 + capacity elements (None stops streaming)."""
        if ring is None:
            st = self.lib.kie_set_token_stream(self.ctx, None, 0)
        else:
            st = self.lib.kie_set_token_stream(self.ctx, _ptr(ring), int(ring.numel()) - 1)
        _check(self.lib, st, self.ctx)
        self._ring = ring  # kept alive while streaming

    @property
    def position(self) -> int:
        return int(self.lib.kie_position(self.ctx))

    def prefill(self, tokens, logits_out=None, smp: Optional[kie_sampling] = None, first_token_out=None):
        """tokens: device int32 tensor [P]. Returns the device int32 [1] tensor of the next token."""
        out = first_token_out if first_token_out is not None else self.torch.empty(1, dtype=self.torch.int32,
                                                                                      device=self.device)
        smp = smp or sampling()
        st = self.lib.kie_prefill(self.ctx, _ptr(tokens), int(tokens.numel()), _ptr(out), _ptr(logits_out),
                                  C.byref(smp))
        _check(self.lib, st, self.ctx)
        return out

    def decode_step(self, token_in, token_out, logits_out=None, smp: Optional[kie_sampling] = None):
        smp = smp or sampling()
        st = self.lib.kie_decode_step(self.ctx, _ptr(token_in), C.byref(smp), _ptr(token_out), _ptr(logits_out))
        _check(self.lib, st, self.ctx)

    def generate(self, first_token, n_steps: int, tokens_out, logits_out=None, forced=None,
                 smp: Optional[kie_sampling] = None):
        smp = smp or sampling()
        st = self.lib.kie_generate(self.ctx, _ptr(first_token), int(n_steps), C.byref(smp), _ptr(forced),
                                   _ptr(tokens_out), _ptr(logits_out))
        _check(self.lib, st, self.ctx)

    def kv_view(self):
        """KV cache as [L][2][nkv][max_seq][hd] int16 bf16 bits."""
        m = self.model
        return self.kv.view(m.n_layers, 2, m.n_kv_heads, self.cfg.max_seq_len, m.head_dim)

    def close(self):
        if getattr(self, "ctx", None):
            self.lib.kie_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_copy(dst, src, nbytes: int, stream) -> None:
    lib = load()
    _check(lib, lib.kie_stream_copy(_ptr(dst), _ptr(src), int(nbytes), C.c_void_p(stream.cuda_stream)))


def stream_read(src, nbytes: int, sink, stream) -> None:
    lib = load()
    _check(lib, lib.kie_stream_read(_ptr(src), int(nbytes), _ptr(sink), C.c_void_p(stream.cuda_stream)))
