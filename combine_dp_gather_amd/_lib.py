"""ctypes declarations of the C ABI in include/moe.h."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_hip.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_CAPACITY, MOE_ERR_HIP, MOE_ERR_SCRATCH_LIMIT = range(6)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_PAD_AUTO, MOE_PAD_MAX_LEN, MOE_PAD_SUM_LEN = 0, 1, 2
MOE_GATE_EXACT, MOE_GATE_FAST = 0, 1
MOE_FP8_ACT_BF16, MOE_FP8_ACT_E4M3 = 0, 1
MOE_ROUTE_SOFTMAX, MOE_ROUTE_GROUPED_SIGMOID = 0, 1
MOE_MAX_REPLICAS = 256

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class GatherLayout(ctypes.Structure):
    _fields_ = [("mode", c_i32), ("num_replicas", c_i32), ("rows", c_i64),
                ("offsets", c_i64 * (MOE_MAX_REPLICAS + 1)), ("sizes", c_i32 * MOE_MAX_REPLICAS)]


class RouteCfg(ctypes.Structure):
    _fields_ = [("kind", c_i32), ("num_experts", c_i32), ("top_k", c_i32), ("n_group", c_i32),
                ("topk_group", c_i32), ("group_topn", c_i32), ("renormalize", c_i32),
                ("gate_mode", c_i32)]


class ExpertMap(ctypes.Structure):
    _fields_ = [("num_logical", c_i32), ("max_rep", c_i32), ("phys_of", c_vp), ("n_rep", c_vp),
                ("first_slot", c_i32), ("num_slots", c_i32)]


class Plan(ctypes.Structure):
    _fields_ = [("counts", c_vp), ("seg_offsets", c_vp), ("sorted_pair", c_vp), ("pair_row", c_vp),
                ("num_rows", c_vp), ("error_flag", c_vp), ("cap", c_i64), ("G", c_i64),
                ("top_k", c_i32), ("num_slots", c_i32), ("align", c_i32), ("seg_stride", c_i32)]


class ExpertWeights(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("fp8_act", c_i32), ("w13", c_vp), ("w2", c_vp), ("s13", c_vp),
                ("s2", c_vp)]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [c_i32]),
    "moe_version": (ctypes.c_char_p, []),
    "moe_gather_layout": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(GatherLayout)]),
    "moe_gather": (c_i32, [ctypes.POINTER(GatherLayout), c_vp, c_i64, c_i32, c_vp, c_vp, c_vp]),
    "moe_scatter": (c_i32, [ctypes.POINTER(GatherLayout), c_vp, c_i64, c_i32, c_vp, c_vp]),
    "moe_expert_load": (c_i32, [c_vp, c_i64, c_i32, ctypes.POINTER(ExpertMap), c_i32, c_vp, c_vp]),
    "moe_physical_to_logical_count": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "moe_eplb_balancedness": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_vp]),
    "moe_eplb_rebalance": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "moe_eplb_logical_to_physical": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "moe_entry_gather": (c_i32, [ctypes.POINTER(GatherLayout), c_vp, c_vp, c_vp, ctypes.c_float, c_i64,
                                 c_i32, c_vp, c_vp, c_vp]),
    "moe_route": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, ctypes.POINTER(RouteCfg),
                          c_vp, c_vp, c_vp, c_vp]),
    "moe_route_from_logits": (c_i32, [c_vp, c_vp, c_i64, c_vp, ctypes.POINTER(RouteCfg), c_vp, c_vp,
                                      c_vp]),
    "moe_dispatch_workspace_size": (c_sz, [c_i64, c_i32, c_i32]),
    "moe_dispatch": (c_i32, [c_vp, c_vp, c_i64, c_i32, c_i64, c_i32, ctypes.POINTER(ExpertMap),
                             ctypes.POINTER(Plan), c_vp, c_vp, c_sz, c_vp]),
    "moe_dispatch_noalloc": (c_i32, [c_vp, c_vp, c_i64, c_i32, c_i64, c_i32, ctypes.POINTER(ExpertMap),
                                     ctypes.POINTER(Plan), c_vp, c_vp]),
    "moe_expert_gemm_fast_path": (c_i32, [c_vp, c_i32, ctypes.POINTER(ExpertWeights), c_i64, c_i64, c_vp, c_vp]),
    "moe_quant_act_fp8": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "moe_expert_gemm_workspace_size": (c_sz, [c_i64, c_i64, c_i64, c_i32, c_i32]),
    "moe_expert_gemm": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan), ctypes.POINTER(ExpertWeights),
                                c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "moe_expert_gemm_up": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan), ctypes.POINTER(ExpertWeights),
                                   c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "moe_expert_gemm_up_gather": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan), ctypes.POINTER(ExpertWeights),
                                          c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "moe_expert_gemm_down": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan),
                                     ctypes.POINTER(ExpertWeights), c_i64, c_i64, c_vp, c_vp, c_sz,
                                     c_vp]),
    "moe_combine": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan), c_vp, c_f32, c_i64, c_vp, c_vp]),
    "moe_combine_scatter": (c_i32, [c_vp, c_i32, ctypes.POINTER(Plan), c_vp, c_f32, c_i64,
                                    ctypes.POINTER(GatherLayout), c_vp, c_vp]),
    "moe_stream_create_cu_masked": (c_i32, [c_vp, ctypes.c_uint32, ctypes.POINTER(c_vp)]),
    "moe_stream_destroy": (c_i32, [c_vp]),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe_hip.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m combine_dp_gather_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        text = load().moe_status_string(status).decode()
        super().__init__(f"{fn}: {text} (status {status})")


def check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status)
