"""Brute-force dense evaluation of a decode MoE layer in NumPy fp64.

A second, independent evaluation used only to pin the oracle on tiny inputs:
it decodes stored codes with lookup tables and, for the E4M3 block scales of
nvfp4 and the fp8 weights, with torch's float8_e4m3fn conversion (the oracle
uses bit formulas),
routes with a stable argsort (the oracle scans), and evaluates EVERY expert on
every row, weighting by a mask that is zero for the experts a row did not
select (the oracle evaluates only the selected ones, slot by slot).
"""
from __future__ import annotations

import numpy as np

# OCP Microscaling Formats v1.0, FP4 E2M1 element values by code 0..15.
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                       -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def act_to_f64(a: np.ndarray, fmt: str) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float64) if fmt == "f32" else bf16_to_f64(a)


def _unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    n, kh = packed.shape
    out = np.empty((n, 2 * kh), np.uint8)
    out[:, 0::2] = packed & 15
    out[:, 1::2] = packed >> 4
    return out


def dense_weight(proj, e: int) -> np.ndarray:
    """Expert e of a synth.Projection as a dense float64 [N, K] matrix."""
    if proj.fmt == "f32":
        return proj.data[e].astype(np.float64)
    if proj.fmt == "bf16":
        return bf16_to_f64(proj.data[e])
    if proj.fmt == "fp8":
        # Each 128 x 128 block's scale tiled over it with a Kronecker product.
        n, k = proj.data[e].shape
        sc = np.kron(proj.scale[e].astype(np.float64), np.ones((128, 128)))[:n, :k]
        return e4m3_to_f64(proj.data[e]) * sc
    q = _unpack_nibbles(proj.data[e])
    if proj.fmt == "aff4":
        s = np.repeat(bf16_to_f64(proj.scale[e]), 64, axis=1)
        b = np.repeat(bf16_to_f64(proj.bias[e]), 64, axis=1)
        return s * q.astype(np.float64) + b
    if proj.fmt == "mxfp4":
        sc = np.repeat(np.ldexp(1.0, proj.scale[e].astype(np.int64) - 127), 32, axis=1)
        return E2M1_TABLE[q] * sc
    if proj.fmt == "nvfp4":
        sc = np.repeat(e4m3_to_f64(proj.scale[e]), 16, axis=1)
        return E2M1_TABLE[q] * sc * float(proj.scale2[e])
    raise ValueError(proj.fmt)


def e4m3_to_f64(b: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 bytes -> float64 through torch's float8_e4m3fn dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def _gelu(v):
    from scipy.stats import norm
    return v * norm.cdf(v)


def round_to_act(v: np.ndarray, fmt: str) -> np.ndarray:
    """Exact values rounded to the activation format (bf16: 8 significant
    bits, to nearest, ties to even)."""
    if fmt == "f32":
        return v.astype(np.float32).astype(np.float64)
    m, e = np.frexp(v)
    q = np.ldexp(1.0, e - 8)
    return np.where(v == 0, 0.0, np.rint(v / q) * q)


def _sqrtsoftplus(v):
    return np.sqrt(np.logaddexp(0.0, v))                 # log(e^0 + e^v)


def _rms_normed(X, w_bits, spec):
    w = act_to_f64(w_bits, spec.act_fmt)
    inv = 1.0 / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + spec.norm_eps)
    return round_to_act(X * w[None, :] * inv, spec.act_fmt)


def dense_forward(layer, x: np.ndarray):
    """Returns (out [m,H], mask-weight matrix [m,E], selected index lists)."""
    spec = layer.spec
    E, k = spec.num_experts, spec.top_k
    X = act_to_f64(x, spec.act_fmt)                      # [m, H]
    Wr = act_to_f64(layer.router, spec.act_fmt)          # [E, H]
    XR = _rms_normed(X, layer.router_norm_w, spec) if spec.router_pre_norm else X
    L = XR @ Wr.T                                        # [m, E]
    bias = 0.0 if layer.expert_bias is None else layer.expert_bias.astype(np.float64)[None, :]
    if spec.routing == "sigmoid_bias":
        key = _sigmoid(L) + bias
    elif spec.routing == "sqrtsoftplus":
        key = _sqrtsoftplus(L) + bias
    else:
        key = L
    m = X.shape[0]
    weights = np.zeros((m, E))
    selected = []
    for r in range(m):
        order = np.argsort(-key[r], kind="stable")[:k]   # ties: lower index first
        selected.append(order)
        if spec.routing == "softmax":
            p = np.exp(L[r] - L[r].max())
            p = p / p.sum()
            wsel = p[order]
        elif spec.routing == "sqrtsoftplus":
            wsel = _sqrtsoftplus(L[r][order])
        else:
            wsel = _sigmoid(L[r][order])
        if spec.norm_topk:
            wsel = wsel / wsel.sum()
        wsel = wsel * spec.routed_scaling_factor
        weights[r, order] = wsel
    mask = np.zeros((m, E), bool)
    for r, order in enumerate(selected):
        mask[r, order] = True
    # The experts' input: the row itself, or RMS-normed (the router above read X).
    XE = _rms_normed(X, layer.pre_norm_w, spec) if spec.pre_expert_norm else X
    out = np.zeros_like(X)
    for e in range(E):
        Wg = dense_weight(layer.gate, e)
        Wu = dense_weight(layer.up, e)
        Wd = dense_weight(layer.down, e)
        if spec.weight_before_ffn:
            U = XE * weights[:, e:e + 1]
            c = mask[:, e].astype(np.float64)
        else:
            U = XE
            c = weights[:, e]
        act = _gelu if spec.activation == "gelu" else _silu
        Y = (act(U @ Wg.T) * (U @ Wu.T)) @ Wd.T
        out += c[:, None] * Y
    if spec.shared:
        Sg = act_to_f64(layer.sh_gate, spec.act_fmt)
        Su = act_to_f64(layer.sh_up, spec.act_fmt)
        Sd = act_to_f64(layer.sh_down, spec.act_fmt)
        act = _gelu if spec.activation == "gelu" else _silu
        ys = (act(XE @ Sg.T) * (XE @ Su.T)) @ Sd.T
        if spec.shared_gated:
            g = _sigmoid(X @ act_to_f64(layer.sh_gate_vec, spec.act_fmt))
            ys = ys * g[:, None]
        out += ys
    return out, weights, selected
