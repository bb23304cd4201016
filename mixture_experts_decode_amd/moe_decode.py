"""ctypes binding of libmoe_decode.so (declared in include/moe_decode.h).

Argument marshalling only: every function here has the name of the C entry
point it calls and passes plain integers (device addresses, sizes, a
hipStream_t) straight through.  A non-OK status raises MoeDecodeError with the
library's thread-local message.  The library must have been built
(``python -m mixture_experts_decode_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_decode.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_decode.h")

# moe_status
MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE",
                4: "MOE_EHIP"}
# moe_format
MOE_F32, MOE_BF16, MOE_AFF4_G64, MOE_MXFP4_B32, MOE_NVFP4_B16, MOE_FP8_B128 = range(6)
FORMATS = {"f32": MOE_F32, "bf16": MOE_BF16, "aff4": MOE_AFF4_G64, "mxfp4": MOE_MXFP4_B32,
           "nvfp4": MOE_NVFP4_B16, "fp8": MOE_FP8_B128}
# moe_routing
MOE_ROUTE_SOFTMAX, MOE_ROUTE_SIGMOID_BIAS, MOE_ROUTE_SIGMOID_LOGIT, MOE_ROUTE_SQRTSOFTPLUS = range(4)
ROUTINGS = {"softmax": MOE_ROUTE_SOFTMAX, "sigmoid_bias": MOE_ROUTE_SIGMOID_BIAS,
            "sigmoid_logit": MOE_ROUTE_SIGMOID_LOGIT, "sqrtsoftplus": MOE_ROUTE_SQRTSOFTPLUS}
# flags
MOE_NORM_TOPK = 1
MOE_WEIGHT_BEFORE_FFN = 2
MOE_SHARED = 4
MOE_SHARED_GATED = 8
MOE_OUT_F32 = 16
MOE_GEGLU = 32
MOE_PRE_EXPERT_NORM = 64
MOE_ROUTER_PRE_NORM = 128


class MoeDecodeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class moe_decode_desc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("max_rows", C.c_int32),
                ("act_fmt", C.c_int32), ("expert_fmt", C.c_int32), ("routing", C.c_int32),
                ("flags", C.c_uint32), ("routed_scaling_factor", C.c_float), ("norm_eps", C.c_float)]


class moe_decode_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "router_w", "expert_bias", "gate_w", "up_w", "down_w", "gate_s", "up_s", "down_s",
        "gate_b", "up_b", "down_b", "sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_vec",
        "gate_scale2", "up_scale2", "down_scale2", "pre_norm_w", "router_norm_w")]


class moe_decode_ws_layout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "logits", "scores", "topk_idx", "topk_w", "row_gate", "sorted_pair", "expert_offsets",
        "pair_to_perm", "active_experts", "active_count", "slot_info", "act", "shared_act", "shared_y",
        "routed_y", "normed_x", "router_x", "sync", "total")]


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mixture_experts_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        st = C.c_int
        vp = C.c_void_p
        L.moe_decode_plan.restype = st
        L.moe_decode_plan.argtypes = [C.POINTER(moe_decode_desc), C.POINTER(vp),
                                      C.POINTER(C.c_size_t)]
        L.moe_decode_plan_destroy.restype = None
        L.moe_decode_plan_destroy.argtypes = [vp]
        L.moe_decode_workspace_layout.restype = st
        L.moe_decode_workspace_layout.argtypes = [vp, C.POINTER(moe_decode_ws_layout)]
        L.moe_decode_workspace_init.restype = st
        L.moe_decode_workspace_init.argtypes = [vp, vp, C.c_size_t, vp]
        fwd = [vp, C.POINTER(moe_decode_weights), vp, C.c_int32, vp, vp, vp, vp, C.c_size_t, vp]
        L.moe_decode_forward.restype = st
        L.moe_decode_forward.argtypes = fwd
        L.moe_decode_forward_noalloc.restype = st
        L.moe_decode_forward_noalloc.argtypes = [vp, C.POINTER(moe_decode_weights), vp, C.c_int32, vp, vp, vp, vp]
        L.moe_decode_forward_timed.restype = st
        L.moe_decode_forward_timed.argtypes = fwd + [C.POINTER(vp), C.c_int32]
        L.moe_decode_num_stages.restype = C.c_int32
        L.moe_decode_num_stages.argtypes = [vp]
        L.moe_decode_stage_name.restype = C.c_char_p
        L.moe_decode_stage_name.argtypes = [vp, C.c_int32]
        L.moe_decode_last_error.restype = C.c_char_p
        L.moe_decode_last_error.argtypes = []
        L.moe_decode_version.restype = C.c_char_p
        L.moe_decode_version.argtypes = []
        L.moe_decode_bench_copy.restype = st
        L.moe_decode_bench_copy.argtypes = [vp, vp, C.c_size_t, vp]
        L.moe_decode_bench_read.restype = st
        L.moe_decode_bench_read.argtypes = [vp, C.c_size_t, vp, vp]
        _lib = L
    return _lib


def header_entry_points() -> list:
    """Names of the functions include/moe_decode.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|void|int32_t|const char \*)\s*(moe_decode_\w+)\(",
                                 text, flags=re.M)))


def moe_decode_last_error() -> str:
    return lib().moe_decode_last_error().decode()


def moe_decode_version() -> str:
    return lib().moe_decode_version().decode()


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeDecodeError(status, moe_decode_last_error())


def moe_decode_plan(desc: moe_decode_desc):
    """-> (plan handle, workspace bytes)."""
    plan = C.c_void_p()
    ws = C.c_size_t()
    _check(lib().moe_decode_plan(C.byref(desc), C.byref(plan), C.byref(ws)))
    return plan.value, ws.value


def moe_decode_plan_destroy(plan) -> None:
    lib().moe_decode_plan_destroy(plan)


def moe_decode_workspace_layout(plan) -> moe_decode_ws_layout:
    out = moe_decode_ws_layout()
    _check(lib().moe_decode_workspace_layout(plan, C.byref(out)))
    return out


def moe_decode_workspace_init(plan, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check(lib().moe_decode_workspace_init(plan, workspace, workspace_bytes, stream))


def moe_decode_forward(plan, weights: moe_decode_weights, x: int, m: int, out: int,
                       idx_out: int | None, w_out: int | None, workspace: int,
                       workspace_bytes: int, stream: int) -> None:
    _check(lib().moe_decode_forward(plan, C.byref(weights), x, m, out, idx_out, w_out,
                                    workspace, workspace_bytes, stream))


def moe_decode_forward_noalloc(plan, weights: moe_decode_weights, x: int, m: int, out: int,
                               idx_out: int | None, w_out: int | None, stream: int) -> None:
    _check(lib().moe_decode_forward_noalloc(plan, C.byref(weights), x, m, out, idx_out, w_out, stream))


def moe_decode_forward_timed(plan, weights: moe_decode_weights, x: int, m: int, out: int,
                             idx_out, w_out, workspace: int, workspace_bytes: int, stream: int,
                             events) -> None:
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().moe_decode_forward_timed(plan, C.byref(weights), x, m, out, idx_out, w_out,
                                          workspace, workspace_bytes, stream, arr, len(events)))


def moe_decode_num_stages(plan) -> int:
    return lib().moe_decode_num_stages(plan)


def moe_decode_stage_name(plan, i: int) -> str:
    return lib().moe_decode_stage_name(plan, i).decode()


def moe_decode_bench_copy(src: int, dst: int, nbytes: int, stream: int) -> None:
    _check(lib().moe_decode_bench_copy(src, dst, nbytes, stream))


def moe_decode_bench_read(src: int, nbytes: int, sink: int, stream: int) -> None:
    _check(lib().moe_decode_bench_read(src, nbytes, sink, stream))
