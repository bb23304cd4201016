"""Seeded synthetic MoE decode layers: the input generator shared by the tests,
the bench and the oracle's callers.

This module only *produces* stored values: Gaussian draws, round-to-nearest-even
to bf16, and the two synthetic 4-bit quantizers that turn a float weight into
stored codes.  It holds none of the layer's arithmetic (no decode, no routing,
no projection): the oracle and the HIP path each decode the stored codes on
their own.

Recipe (every array has its own counter-keyed NumPy PCG64 stream, so any one
of them can be regenerated alone and the experts can be drawn in parallel):

    stream key [seed, 0, 0]      router weight  [E, H]
    stream key [seed, 1, 0]      expert_bias    [E]        (sigmoid+bias routing)
    stream key [seed, 2+j, e]    expert e, projection j (0 gate [I,H], 1 up [I,H], 2 down [H,I])
    stream key [seed, 5, j]      shared expert projection j (Is instead of I)
    stream key [seed, 6, 0]      shared-expert gate vector w_g [H]
    stream key [seed, 7, b]      activation block b: x [max_rows, H]
    stream key [seed, 8, 0]      pre-expert norm weight [H]: 1 + z * 0.1
    stream key [seed, 9, 0]      router pre-norm weight [H]: 1 + z * 0.1

Each weight is ``f32(z * std)`` with ``z`` a float32 standard normal, then
stored as f32, bf16 (RNE) or quantized (aff4 / mxfp4 / nvfp4 below).  ``x`` is
``f32(z * x_std)`` stored in the activation format.

Formats (stored codes):
  * ``bf16``: uint16 bit patterns.
  * ``aff4``: 4-bit affine, group 64 along K.  ``packed [N, K/2]`` uint8 with
    element 2t in the low nibble of byte t, ``scale [N, K/64]`` and
    ``bias [N, K/64]`` bf16 bit patterns; the value is ``scale*q + bias``.
    Quantizer: per group ``s = bf16(max-min)/15``, ``b = bf16(min)``,
    ``q = clamp(rint((w-b)/s), 0, 15)`` (s = 0 -> s = 1, q = 0).
  * ``mxfp4``: OCP MX E2M1 codes, low nibble first, ``packed [N, K/2]`` uint8
    and one E8M0 byte per 32 elements, ``scale [N, K/32]``.  Quantizer:
    ``e = clamp(floor(log2(amax)) - 2 + 127, 1, 254)``, code = nearest E2M1
    value of ``w / 2^(e-127)``, ties to the even code, saturating at 6.
  * ``nvfp4``: E2M1 codes packed like mxfp4, one OCP E4M3 byte per 16
    elements, ``scale [N, K/16]``, and one float32 second-level scale per
    expert projection, ``scale2 [E]``.  Quantizer (per projection):
    ``s2 = f32(amax / (6 * 448))`` (1 if amax = 0); per block the E4M3 value
    nearest ``amax_block / (6 * s2)`` (ties to the even code); codes = nearest
    E2M1 value of ``w / (E4M3(scale) * s2)``, ties to the even code,
    saturating at 6 (all 0 where the block scale is 0).
  * ``fp8``: one OCP E4M3 byte per element, ``data [N, K]`` uint8, and one
    float32 scale per 128 x 128 block, ``scale [ceil(N/128), ceil(K/128)]``
    (the last blocks ragged).  Quantizer (per block): ``s = f32(amax / 448)``
    (1 if amax = 0); code = nearest E4M3 value of ``w / s``, ties to the even
    code, saturating at 448, sign in bit 7.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

ACT_FORMATS = ("f32", "bf16")
EXPERT_FORMATS = ("f32", "bf16", "aff4", "mxfp4", "nvfp4", "fp8")
ROUTINGS = ("softmax", "sigmoid_bias", "sigmoid_logit", "sqrtsoftplus")
ACTIVATIONS = ("silu", "gelu")

# Group sizes of the 4-bit formats along the reduction dimension K.
AFF4_GROUP = 64
MXFP4_BLOCK = 32
NVFP4_BLOCK = 16
# The fp8 scale block: FP8_BLOCK x FP8_BLOCK elements of [N, K].
FP8_BLOCK = 128


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape, formats and routing flags of one decode MoE layer."""

    name: str
    hidden: int
    num_experts: int
    top_k: int
    inter: int
    shared_inter: int = 0
    act_fmt: str = "bf16"
    expert_fmt: str = "bf16"
    routing: str = "softmax"
    norm_topk: bool = True
    weight_before_ffn: bool = False
    shared: bool = False
    shared_gated: bool = False
    routed_scaling_factor: float = 1.0
    activation: str = "silu"        # expert activation: "silu" (SwiGLU) or "gelu" (GeGLU)
    pre_expert_norm: bool = False   # experts read the row RMS-normed (weight pre_norm_w); router: raw
    router_pre_norm: bool = False   # the router reads the row RMS-normed (weight router_norm_w)
    route_bias: Optional[bool] = None  # an expert bias [E] for selection (default: sigmoid_bias only)
    norm_eps: float = 1e-6
    w_std: float = 0.02
    x_std: float = 1.0
    bias_std: float = 0.1
    rows: tuple = (1,)

    @property
    def max_rows(self) -> int:
        return max(self.rows)

    @property
    def biased(self) -> bool:
        """Whether the layer has an expert bias (required by sigmoid_bias)."""
        return self.routing == "sigmoid_bias" if self.route_bias is None else bool(self.route_bias)

    def replace(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


# The six workloads: shapes and routing of real decode MoE layers, with
# synthetic seeded weights.  The nvfp4 and fp8 ones are the mxfp4 layer's
# shape with the experts stored as NVFP4 or block-scaled FP8 (the formats of
# that model family's NVFP4 and FP8 checkpoints).
WORKLOADS = {
    "tiny_f32": LayerSpec(
        name="tiny_f32", hidden=64, num_experts=8, top_k=2, inter=32,
        act_fmt="f32", expert_fmt="f32", routing="softmax", norm_topk=True,
        w_std=0.1, rows=(1,)),
    "qwen3_30b_a3b_bf16": LayerSpec(
        name="qwen3_30b_a3b_bf16", hidden=2048, num_experts=128, top_k=8, inter=768,
        act_fmt="bf16", expert_fmt="bf16", routing="softmax", norm_topk=True,
        rows=(1, 2, 4, 8)),
    "lfm2_8b_a1b_aff4": LayerSpec(
        name="lfm2_8b_a1b_aff4", hidden=2048, num_experts=32, top_k=4, inter=1792,
        act_fmt="bf16", expert_fmt="aff4", routing="sigmoid_bias", norm_topk=True,
        routed_scaling_factor=1.0, rows=(1, 4, 8)),
    "qwen35_35b_a3b_mxfp4": LayerSpec(
        name="qwen35_35b_a3b_mxfp4", hidden=2048, num_experts=256, top_k=8, inter=512,
        shared_inter=512, act_fmt="bf16", expert_fmt="mxfp4", routing="softmax",
        norm_topk=True, shared=True, shared_gated=True, rows=(1, 8, 16)),
    "qwen35_35b_a3b_nvfp4": LayerSpec(
        name="qwen35_35b_a3b_nvfp4", hidden=2048, num_experts=256, top_k=8, inter=512,
        shared_inter=512, act_fmt="bf16", expert_fmt="nvfp4", routing="softmax",
        norm_topk=True, shared=True, shared_gated=True, rows=(1, 8, 16)),
    "qwen35_35b_a3b_fp8": LayerSpec(
        name="qwen35_35b_a3b_fp8", hidden=2048, num_experts=256, top_k=8, inter=512,
        shared_inter=512, act_fmt="bf16", expert_fmt="fp8", routing="softmax",
        norm_topk=True, shared=True, shared_gated=True, rows=(1, 8, 16)),
    "llama4_wbf_bf16": LayerSpec(
        name="llama4_wbf_bf16", hidden=5120, num_experts=16, top_k=1, inter=8192,
        shared_inter=8192, act_fmt="bf16", expert_fmt="bf16", routing="sigmoid_logit",
        norm_topk=False, weight_before_ffn=True, shared=True, shared_gated=False,
        rows=(1, 8, 32)),
}


# ----------------------------------------------------------------------------
# Stored-value encoders (generator side only).
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even, and return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    # Used only to feed the quantizers their own rounded scale/bias values.
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_aff4(w: np.ndarray):
    """4-bit affine quantizer, group 64 along the last axis -> (packed, scale, bias)."""
    n, k = w.shape
    assert k % AFF4_GROUP == 0
    g = w.reshape(n, k // AFF4_GROUP, AFF4_GROUP).astype(np.float32)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    s_bits = f32_to_bf16_bits((mx - mn) / np.float32(15.0))
    b_bits = f32_to_bf16_bits(mn)
    s = _bf16_bits_to_f32(s_bits).astype(np.float64)
    zero = s == 0.0
    s_bits = np.where(zero, np.uint16(0x3F80), s_bits)  # bf16 1.0
    s = np.where(zero, 1.0, s)
    b = _bf16_bits_to_f32(b_bits).astype(np.float64)
    q = np.rint((g.astype(np.float64) - b[..., None]) / s[..., None])
    q = np.clip(q, 0, 15)
    q = np.where(zero[..., None], 0, q).astype(np.uint8).reshape(n, k)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, s_bits.astype(np.uint16), b_bits.astype(np.uint16)


# Decision thresholds between neighbouring E2M1 magnitudes
# {0, 0.5, 1, 1.5, 2, 3, 4, 6} (codes 0..7).
_E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def quantize_mxfp4(w: np.ndarray):
    """MXFP4 quantizer, E8M0 scale per 32 along the last axis -> (packed, scale)."""
    n, k = w.shape
    assert k % MXFP4_BLOCK == 0
    g = w.reshape(n, k // MXFP4_BLOCK, MXFP4_BLOCK).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore"):
        lg = np.floor(np.log2(np.where(amax > 0, amax, 1e-300)))
    e = np.clip(lg - 2 + 127, 1, 254).astype(np.int64)
    scaled = g / np.ldexp(1.0, e - 127)[..., None]
    a = np.abs(scaled)
    code = np.searchsorted(_E2M1_MIDPOINTS, a, side="left")
    tie = (code < 7) & (a == _E2M1_MIDPOINTS[np.minimum(code, 6)])
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    code = np.minimum(code, 7)
    code = code | np.where(scaled < 0, 8, 0)
    code = code.astype(np.uint8).reshape(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, e.astype(np.uint8)


def _e4m3_positive_values() -> np.ndarray:
    """Values of the E4M3 bytes 0x00..0x7E (the non-negative, non-NaN codes)."""
    b = np.arange(0x7F)
    ex, man = b >> 3, b & 7
    return np.where(ex == 0, np.ldexp(man / 8.0, -6), np.ldexp(1.0 + man / 8.0, ex - 7))


_E4M3_POS = _e4m3_positive_values()
_E4M3_MIDPOINTS = 0.5 * (_E4M3_POS[1:] + _E4M3_POS[:-1])


def _nearest_code(a: np.ndarray, midpoints: np.ndarray) -> np.ndarray:
    """Index of the nearest table value for a >= 0 (ties to the even index,
    saturating at the last one)."""
    code = np.searchsorted(midpoints, a, side="left")
    last = len(midpoints)
    tie = (code < last) & (a == midpoints[np.minimum(code, last - 1)])
    code = np.where(tie & (code % 2 == 1), code + 1, code)
    return np.minimum(code, last)


def quantize_nvfp4(w: np.ndarray):
    """NVFP4 quantizer -> (packed [N, K/2], E4M3 scale bytes [N, K/16], float32 s2)."""
    n, k = w.shape
    assert k % NVFP4_BLOCK == 0
    w64 = w.astype(np.float64)
    amax = float(np.abs(w64).max()) if w64.size else 0.0
    s2 = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    if s2 == 0:
        s2 = np.float32(1.0)
    g = w64.reshape(n, k // NVFP4_BLOCK, NVFP4_BLOCK)
    target = np.abs(g).max(axis=2) / (6.0 * float(s2))
    sc = _nearest_code(np.minimum(target, 448.0), _E4M3_MIDPOINTS).astype(np.uint8)
    denom = _E4M3_POS[sc] * float(s2)
    with np.errstate(divide="ignore", invalid="ignore"):
        scaled = np.where(denom[..., None] > 0, g / denom[..., None], 0.0)
    code = _nearest_code(np.abs(scaled), _E2M1_MIDPOINTS)
    code = code | np.where(scaled < 0, 8, 0)
    code = code.astype(np.uint8).reshape(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc, s2


def quantize_fp8(w: np.ndarray):
    """FP8 quantizer -> (E4M3 bytes [N, K], float32 scales [ceil(N/128), ceil(K/128)])."""
    n, k = w.shape
    nb, kb = -(-n // FP8_BLOCK), -(-k // FP8_BLOCK)
    w64 = w.astype(np.float64)
    scale = np.ones((nb, kb), np.float32)
    codes = np.zeros((n, k), np.uint8)
    for bi in range(nb):
        for bj in range(kb):
            blk = w64[bi * FP8_BLOCK:(bi + 1) * FP8_BLOCK, bj * FP8_BLOCK:(bj + 1) * FP8_BLOCK]
            amax = float(np.abs(blk).max()) if blk.size else 0.0
            s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
            if s == 0:
                s = np.float32(1.0)
            scale[bi, bj] = s
            scaled = blk / float(s)
            c = _nearest_code(np.abs(scaled), _E4M3_MIDPOINTS) | np.where(scaled < 0, 0x80, 0)
            codes[bi * FP8_BLOCK:(bi + 1) * FP8_BLOCK, bj * FP8_BLOCK:(bj + 1) * FP8_BLOCK] = c
    return codes, scale


# ----------------------------------------------------------------------------
# Layer generation.
# ----------------------------------------------------------------------------

def _rng(seed: int, stream: int, index: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(index)])


def _draw(seed, stream, index, shape, std) -> np.ndarray:
    z = _rng(seed, stream, index).standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    return z


def _store_act(w: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f32":
        return np.ascontiguousarray(w, dtype=np.float32)
    if fmt == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(fmt)


@dataclasses.dataclass
class Projection:
    """All E experts' copies of one projection, stacked on axis 0.

    ``data`` is [E, N, K] (f32 / bf16 bits / fp8 bytes) or [E, N, K/2] packed
    4-bit codes; ``scale`` / ``bias`` are [E, N, K/G] (fp8: [E, ceil(N/128),
    ceil(K/128)] float32) or None; ``scale2`` is the nvfp4
    second-level scale of each expert's copy, [E] float32, else None.
    """

    fmt: str
    n: int
    k: int
    data: np.ndarray
    scale: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None
    scale2: Optional[np.ndarray] = None


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    seed: int
    router: np.ndarray                  # [E, H] act_fmt
    expert_bias: Optional[np.ndarray]   # [E] f32
    gate: Projection                    # [E, I, H]
    up: Projection                      # [E, I, H]
    down: Projection                    # [E, H, I]
    sh_gate: Optional[np.ndarray]       # [Is, H] act_fmt
    sh_up: Optional[np.ndarray]         # [Is, H] act_fmt
    sh_down: Optional[np.ndarray]       # [H, Is] act_fmt
    sh_gate_vec: Optional[np.ndarray]   # [H] act_fmt
    pre_norm_w: Optional[np.ndarray] = None   # [H] act_fmt (pre_expert_norm)
    router_norm_w: Optional[np.ndarray] = None   # [H] act_fmt (router_pre_norm)

    def x(self, block: int = 0, rows: Optional[int] = None) -> np.ndarray:
        return make_x(self.spec, self.seed, block, rows)

    def expert_bytes(self) -> int:
        """Stored bytes of one routed expert (gate + up + down)."""
        tot = 0
        for p in (self.gate, self.up, self.down):
            tot += p.data[0].nbytes
            if p.scale is not None:
                tot += p.scale[0].nbytes
            if p.bias is not None:
                tot += p.bias[0].nbytes
            if p.scale2 is not None:
                tot += p.scale2[0].nbytes
        return tot


def _alloc_projection(fmt: str, e: int, n: int, k: int) -> Projection:
    if fmt == "f32":
        return Projection(fmt, n, k, np.empty((e, n, k), np.float32))
    if fmt == "bf16":
        return Projection(fmt, n, k, np.empty((e, n, k), np.uint16))
    if fmt == "aff4":
        g = k // AFF4_GROUP
        return Projection(fmt, n, k, np.empty((e, n, k // 2), np.uint8),
                          np.empty((e, n, g), np.uint16), np.empty((e, n, g), np.uint16))
    if fmt == "mxfp4":
        return Projection(fmt, n, k, np.empty((e, n, k // 2), np.uint8),
                          np.empty((e, n, k // MXFP4_BLOCK), np.uint8))
    if fmt == "nvfp4":
        return Projection(fmt, n, k, np.empty((e, n, k // 2), np.uint8),
                          np.empty((e, n, k // NVFP4_BLOCK), np.uint8),
                          scale2=np.empty((e,), np.float32))
    if fmt == "fp8":
        return Projection(fmt, n, k, np.empty((e, n, k), np.uint8),
                          np.empty((e, -(-n // FP8_BLOCK), -(-k // FP8_BLOCK)), np.float32))
    raise ValueError(fmt)


def _fill_expert(proj: Projection, e: int, w: np.ndarray) -> None:
    if proj.fmt == "f32":
        proj.data[e] = w
    elif proj.fmt == "bf16":
        proj.data[e] = f32_to_bf16_bits(w)
    elif proj.fmt == "aff4":
        proj.data[e], proj.scale[e], proj.bias[e] = quantize_aff4(w)
    elif proj.fmt == "mxfp4":
        proj.data[e], proj.scale[e] = quantize_mxfp4(w)
    elif proj.fmt == "nvfp4":
        proj.data[e], proj.scale[e], proj.scale2[e] = quantize_nvfp4(w)
    elif proj.fmt == "fp8":
        proj.data[e], proj.scale[e] = quantize_fp8(w)


def check_spec(spec: LayerSpec) -> None:
    if spec.act_fmt not in ACT_FORMATS or spec.expert_fmt not in EXPERT_FORMATS:
        raise ValueError("bad format")
    if spec.routing not in ROUTINGS:
        raise ValueError("bad routing")
    if spec.activation not in ACTIVATIONS:
        raise ValueError("bad activation")
    if spec.routing == "sigmoid_bias" and not spec.biased:
        raise ValueError("sigmoid_bias routing needs the expert bias")
    if spec.biased and spec.routing not in ("sigmoid_bias", "sqrtsoftplus"):
        raise ValueError("an expert bias serves sigmoid_bias and sqrtsoftplus routing only")
    if spec.expert_fmt == "aff4" and (spec.hidden % AFF4_GROUP or spec.inter % AFF4_GROUP):
        raise ValueError("aff4 needs H and I multiples of 64")
    if spec.expert_fmt == "mxfp4" and (spec.hidden % MXFP4_BLOCK or spec.inter % MXFP4_BLOCK):
        raise ValueError("mxfp4 needs H and I multiples of 32")
    if spec.expert_fmt == "nvfp4" and (spec.hidden % 32 or spec.inter % 32):
        raise ValueError("nvfp4 needs H and I multiples of 32")


def make_layer(spec: LayerSpec, seed: int = 0, threads: Optional[int] = None) -> Layer:
    """Generate every stored array of one layer from ``seed`` (recipe: module doc)."""
    check_spec(spec)
    H, E, I, Is = spec.hidden, spec.num_experts, spec.inter, spec.shared_inter
    router = _store_act(_draw(seed, 0, 0, (E, H), spec.w_std), spec.act_fmt)
    bias = None
    if spec.biased:
        bias = _draw(seed, 1, 0, (E,), spec.bias_std).astype(np.float32)
    gate = _alloc_projection(spec.expert_fmt, E, I, H)
    up = _alloc_projection(spec.expert_fmt, E, I, H)
    down = _alloc_projection(spec.expert_fmt, E, H, I)
    projs = (gate, up, down)

    def one(task):
        e, j = task
        p = projs[j]
        _fill_expert(p, e, _draw(seed, 2 + j, e, (p.n, p.k), spec.w_std))

    tasks = [(e, j) for e in range(E) for j in range(3)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr > 1 and len(tasks) > 1:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, tasks))
    else:
        for t in tasks:
            one(t)

    sh_gate = sh_up = sh_down = sh_vec = None
    if spec.shared:
        sh_gate = _store_act(_draw(seed, 5, 0, (Is, H), spec.w_std), spec.act_fmt)
        sh_up = _store_act(_draw(seed, 5, 1, (Is, H), spec.w_std), spec.act_fmt)
        sh_down = _store_act(_draw(seed, 5, 2, (H, Is), spec.w_std), spec.act_fmt)
        if spec.shared_gated:
            sh_vec = _store_act(_draw(seed, 6, 0, (H,), spec.w_std), spec.act_fmt)
    norm_w = rnorm_w = None
    if spec.pre_expert_norm:
        norm_w = _store_act(_draw(seed, 8, 0, (H,), 0.1) + np.float32(1.0), spec.act_fmt)
    if spec.router_pre_norm:
        rnorm_w = _store_act(_draw(seed, 9, 0, (H,), 0.1) + np.float32(1.0), spec.act_fmt)
    return Layer(spec, seed, router, bias, gate, up, down, sh_gate, sh_up, sh_down, sh_vec, norm_w, rnorm_w)


def make_x(spec: LayerSpec, seed: int = 0, block: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """Activation block ``block``: [rows, H] in the activation format (first rows of the block)."""
    n = spec.max_rows if rows is None else rows
    full = _draw(seed, 7, block, (max(n, spec.max_rows), spec.hidden), spec.x_std)
    return _store_act(full[:n], spec.act_fmt)
