"""CPU oracle of the batch-1 decoder step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this package. It does not
import the GPU package and the GPU package does not import it.
"""
from .oracle import (OracleModel, build, lib_path, gemv, rmsnorm, rope, attend, silu, argmax,
                     topk_sample, splitmix64, uniform, f32_to_bf16, bf16_to_f32, set_threads,
                     set_gemv_order, full_recompute, moe_route, e4m3_to_f32, gemv_e4m3)
from . import bytes_model

__all__ = ["OracleModel", "build", "lib_path", "gemv", "rmsnorm", "rope", "attend", "silu", "argmax",
           "topk_sample", "splitmix64", "uniform", "f32_to_bf16", "bf16_to_f32", "set_threads",
           "set_gemv_order", "full_recompute", "moe_route", "e4m3_to_f32", "gemv_e4m3", "bytes_model"]
