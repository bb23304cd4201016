"""The oracle: plain fp64 CPU evaluation of the decode MoE layer (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the HIP product path
never calls it and shares no code with it (only the seeded input generator
``mixture_experts_decode_amd.synth`` feeds both).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
values the pages print, closed forms, special cases and a NumPy brute-force
dense evaluation (``tests/dense_ref.py``).  Nothing is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

FMT = {"f32": 0, "bf16": 1, "aff4": 2, "mxfp4": 3, "nvfp4": 4, "fp8": 5}
ROUTING = {"softmax": 0, "sigmoid_bias": 1, "sigmoid_logit": 2, "sqrtsoftplus": 3}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into ``libmoe_oracle.so``."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-fopenmp", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "hidden", "num_experts", "top_k", "inter", "shared_inter", "act_fmt", "expert_fmt",
        "routing", "norm_topk", "weight_before_ffn", "shared", "shared_gated")] + [
        ("routed_scaling_factor", C.c_double), ("geglu", C.c_int32), ("pre_norm", C.c_int32),
        ("norm_eps", C.c_double), ("router_pre_norm", C.c_int32)]


_PP = C.POINTER(C.c_void_p)


class _Weights(C.Structure):
    _fields_ = [("router", C.c_void_p), ("expert_bias", C.c_void_p)] + [
        (n, _PP) for n in ("gate", "up", "down", "gate_s", "up_s", "down_s",
                           "gate_b", "up_b", "down_b")] + [
        (n, C.c_void_p) for n in ("sh_gate", "sh_up", "sh_down", "sh_gate_vec", "pre_norm_w",
                                  "router_norm_w")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = C.CDLL(LIB_PATH)
        L.orc_forward.restype = C.c_int32
        L.orc_forward.argtypes = [C.POINTER(_Desc), C.POINTER(_Weights), C.c_void_p, C.c_int32,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_sqrtsoftplus.restype = C.c_double
        L.orc_sqrtsoftplus.argtypes = [C.c_double]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [C.c_uint8]
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [C.c_int32]
        L.orc_get_threads.restype = C.c_int32
        L.orc_get_threads.argtypes = []
        L.orc_round_act.restype = C.c_double
        L.orc_round_act.argtypes = [C.c_int32, C.c_double]
        L.orc_decode_act.restype = C.c_double
        L.orc_decode_act.argtypes = [C.c_int32, C.c_void_p, C.c_int64]
        L.orc_decode_row.restype = None
        L.orc_decode_row.argtypes = [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                     C.c_int32, C.c_void_p]
        L.orc_routed_slot.restype = None
        L.orc_routed_slot.argtypes = [C.c_void_p, C.c_int32, C.c_double, C.c_int32, C.c_void_p,
                                      C.c_void_p]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [C.POINTER(_Desc), C.POINTER(_Weights), C.c_void_p,
                                        C.c_void_p]
        L.orc_select.restype = None
        L.orc_select.argtypes = [C.POINTER(_Desc), C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p]
        L.orc_sort_pairs.restype = None
        L.orc_sort_pairs.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def desc_of(spec) -> _Desc:
    return _Desc(spec.hidden, spec.num_experts, spec.top_k, spec.inter,
                 spec.shared_inter if spec.shared else 0, FMT[spec.act_fmt],
                 FMT[spec.expert_fmt], ROUTING[spec.routing], int(spec.norm_topk),
                 int(spec.weight_before_ffn), int(spec.shared), int(spec.shared_gated),
                 float(spec.routed_scaling_factor), int(spec.activation == "gelu"),
                 int(spec.pre_expert_norm), float(spec.norm_eps), int(spec.router_pre_norm))


def _table(arr: Optional[np.ndarray]):
    """[E, ...] stacked array -> C array of E host pointers (or NULL)."""
    if arr is None:
        return None
    assert arr.flags["C_CONTIGUOUS"]
    E = arr.shape[0]
    stride = arr[0].nbytes
    base = arr.ctypes.data
    return (C.c_void_p * E)(*[base + e * stride for e in range(E)])


class _Bound:
    """Keeps the ctypes pointer tables of one layer alive."""

    def __init__(self, layer):
        self.layer = layer
        self.desc = desc_of(layer.spec)
        self.keep = []
        w = _Weights()
        w.router = _ptr(layer.router)
        w.expert_bias = _ptr(layer.expert_bias)
        for name in ("gate", "up", "down"):
            p = getattr(layer, name)
            # nvfp4: the "_b" entry of expert e points to its second-level scale.
            second = p.scale2 if p.scale2 is not None else p.bias
            for suffix, arr in (("", p.data), ("_s", p.scale), ("_b", second)):
                t = _table(arr)
                self.keep.append(t)
                setattr(w, name + suffix, C.cast(t, _PP) if t is not None else None)
        w.sh_gate = _ptr(layer.sh_gate)
        w.sh_up = _ptr(layer.sh_up)
        w.sh_down = _ptr(layer.sh_down)
        w.sh_gate_vec = _ptr(layer.sh_gate_vec)
        w.pre_norm_w = _ptr(layer.pre_norm_w)
        w.router_norm_w = _ptr(layer.router_norm_w)
        self.weights = w


_bound_cache: dict = {}


def _bound(layer) -> _Bound:
    key = id(layer)
    b = _bound_cache.get(key)
    if b is None or b.layer is not layer:
        b = _Bound(layer)
        _bound_cache.clear()
        _bound_cache[key] = b
    return b


@dataclasses.dataclass
class OracleResult:
    out: np.ndarray      # [m, H] float64
    idx: np.ndarray      # [m, k] int32
    w: np.ndarray        # [m, k] float64
    logits: np.ndarray   # [m, E] float64
    margin: np.ndarray   # [m] float64


def forward(layer, x: np.ndarray) -> OracleResult:
    """The layer on the rows of ``x`` ([m, H], activation format)."""
    spec = layer.spec
    x = np.ascontiguousarray(x)
    m = x.shape[0]
    assert x.shape[1] == spec.hidden
    out = np.zeros((m, spec.hidden), np.float64)
    idx = np.zeros((m, spec.top_k), np.int32)
    w = np.zeros((m, spec.top_k), np.float64)
    logits = np.zeros((m, spec.num_experts), np.float64)
    margin = np.zeros((m,), np.float64)
    b = _bound(layer)
    rc = lib().orc_forward(C.byref(b.desc), C.byref(b.weights), _ptr(x), m, _ptr(out),
                           _ptr(idx), _ptr(w), _ptr(logits), _ptr(margin))
    if rc != 0:
        raise ValueError("oracle rejected the layer description")
    return OracleResult(out, idx, w, logits, margin)


def router_logits(layer, x_row: np.ndarray) -> np.ndarray:
    b = _bound(layer)
    x_row = np.ascontiguousarray(x_row)
    out = np.zeros(layer.spec.num_experts, np.float64)
    lib().orc_router_logits(C.byref(b.desc), C.byref(b.weights), _ptr(x_row), _ptr(out))
    return out


def select(spec, logits: np.ndarray, expert_bias: Optional[np.ndarray] = None):
    """(idx[k], w[k], margin) of one row from its logits."""
    d = desc_of(spec)
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    bias = None if expert_bias is None else np.ascontiguousarray(expert_bias, dtype=np.float32)
    idx = np.zeros(spec.top_k, np.int32)
    w = np.zeros(spec.top_k, np.float64)
    mg = np.zeros(1, np.float64)
    lib().orc_select(C.byref(d), _ptr(bias), _ptr(logits), _ptr(idx), _ptr(w), _ptr(mg))
    return idx, w, float(mg[0])


def sort_pairs(idx: np.ndarray, num_experts: int) -> dict:
    """Stable counting sort of the [m, k] pairs by expert."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    m, k = idx.shape
    te = m * k
    sp = np.zeros(te, np.int32)
    off = np.zeros(num_experts + 1, np.int32)
    p2p = np.zeros(te, np.int32)
    act = np.zeros(max(1, min(te, num_experts)), np.int32)
    cnt = np.zeros(1, np.int32)
    lib().orc_sort_pairs(m, k, num_experts, _ptr(idx), _ptr(sp), _ptr(off), _ptr(p2p),
                         _ptr(act), _ptr(cnt))
    n = int(cnt[0])
    return {"sorted_pair": sp, "expert_offsets": off, "pair_to_perm": p2p,
            "active_experts": act[:n].copy(), "active_count": n}


def decode_row(fmt: str, w: np.ndarray, s: Optional[np.ndarray], b: Optional[np.ndarray],
               K: int, n: int) -> np.ndarray:
    out = np.zeros(K, np.float64)
    lib().orc_decode_row(FMT[fmt], _ptr(np.ascontiguousarray(w)),
                         _ptr(None if s is None else np.ascontiguousarray(s)),
                         _ptr(None if b is None else np.ascontiguousarray(b)), K, n, _ptr(out))
    return out


def sqrtsoftplus(v: float) -> float:
    """The sqrt-softplus router score sqrt(log(1 + e^v))."""
    return float(lib().orc_sqrtsoftplus(float(v)))


def e4m3_value(b: int) -> float:
    """One OCP FP8 E4M3 byte as a float (NaN for the NaN codes)."""
    return float(lib().orc_e4m3_value(int(b)))


def set_threads(n: int) -> None:
    """Threads (OpenMP) over each projection's output neurons; results do not
    depend on the count."""
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def round_act(fmt: str, v: float) -> float:
    """v rounded to the activation format ("f32", or "bf16": to nearest, ties to even)."""
    return float(lib().orc_round_act(FMT[fmt], float(v)))


def decode_act(fmt: str, a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    L = lib()
    return np.array([L.orc_decode_act(FMT[fmt], _ptr(a), i) for i in range(a.size)])


def routed_slot(x, w: float, before_ffn: bool):
    x = np.ascontiguousarray(x, dtype=np.float64)
    xo = np.zeros_like(x)
    wo = np.zeros(1, np.float64)
    lib().orc_routed_slot(_ptr(x), x.size, float(w), int(before_ffn), _ptr(xo), _ptr(wo))
    return xo, float(wo[0])
