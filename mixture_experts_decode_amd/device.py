"""Device-side copy of a layer: uploads stored weights with torch, builds the
per-expert pointer tables and the plan/workspace, and calls the C ABI.

torch supplies device memory and the current HIP stream only; the forward
itself is ``moe_decode.moe_decode_forward`` (libmoe_decode.so).
"""
from __future__ import annotations

import weakref
from typing import Optional

import numpy as np
import torch

from . import moe_decode as md
from .synth import Layer, LayerSpec


def desc_of(spec: LayerSpec, max_rows: Optional[int] = None, out_f32: bool = False) -> md.moe_decode_desc:
    flags = 0
    if spec.norm_topk:
        flags |= md.MOE_NORM_TOPK
    if spec.weight_before_ffn:
        flags |= md.MOE_WEIGHT_BEFORE_FFN
    if spec.shared:
        flags |= md.MOE_SHARED
    if spec.shared_gated:
        flags |= md.MOE_SHARED_GATED
    if out_f32:
        flags |= md.MOE_OUT_F32
    if spec.activation == "gelu":
        flags |= md.MOE_GEGLU
    if spec.pre_expert_norm:
        flags |= md.MOE_PRE_EXPERT_NORM
    if spec.router_pre_norm:
        flags |= md.MOE_ROUTER_PRE_NORM
    return md.moe_decode_desc(
        hidden=spec.hidden, num_experts=spec.num_experts, top_k=spec.top_k, inter=spec.inter,
        shared_inter=spec.shared_inter if spec.shared else 0,
        max_rows=max_rows or spec.max_rows, act_fmt=md.FORMATS[spec.act_fmt],
        expert_fmt=md.FORMATS[spec.expert_fmt], routing=md.ROUTINGS[spec.routing], flags=flags,
        routed_scaling_factor=spec.routed_scaling_factor, norm_eps=spec.norm_eps)


def to_device(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    """Stored array -> device tensor with the same bytes (uint16 travels as int16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def act_dtype(spec: LayerSpec):
    return torch.float32 if spec.act_fmt == "f32" else torch.int16


def x_to_device(spec: LayerSpec, x: np.ndarray, device="cuda") -> torch.Tensor:
    return to_device(x, device)


class _Copy:
    """One full set of device weights with its pointer tables."""

    def __init__(self, tensors: dict, E: int, device):
        self.t = tensors
        self.tables = {}
        for name in ("gate", "up", "down"):
            for suffix in ("", "_s", "_b"):
                arr = tensors.get(name + suffix)
                if arr is None:
                    continue
                stride = arr[0].numel() * arr.element_size()
                base = arr.data_ptr()
                self.tables[name + suffix] = torch.tensor(
                    [base + e * stride for e in range(E)], dtype=torch.int64, device=device)

        def p(t):
            return None if t is None else t.data_ptr()

        self.weights = md.moe_decode_weights(
            router_w=p(tensors["router"]), expert_bias=p(tensors.get("bias")),
            gate_w=p(self.tables["gate"]), up_w=p(self.tables["up"]), down_w=p(self.tables["down"]),
            gate_s=p(self.tables.get("gate_s")), up_s=p(self.tables.get("up_s")),
            down_s=p(self.tables.get("down_s")), gate_b=p(self.tables.get("gate_b")),
            up_b=p(self.tables.get("up_b")), down_b=p(self.tables.get("down_b")),
            sh_gate_w=p(tensors.get("sh_gate")), sh_up_w=p(tensors.get("sh_up")),
            sh_down_w=p(tensors.get("sh_down")), sh_gate_vec=p(tensors.get("sh_gate_vec")),
            gate_scale2=p(tensors.get("gate_s2")), up_scale2=p(tensors.get("up_s2")),
            down_scale2=p(tensors.get("down_s2")), pre_norm_w=p(tensors.get("pre_norm_w")),
            router_norm_w=p(tensors.get("router_norm_w")))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.t.values() if t is not None)


class DeviceLayer:
    """A layer resident on one GPU, ``copies`` times (distinct device memory
    per copy, so consecutive calls can be kept out of the caches)."""

    def __init__(self, layer: Layer, max_rows: Optional[int] = None, out_f32: bool = False,
                 device="cuda", copies: int = 1):
        spec = layer.spec
        self.spec = spec
        self.device = torch.device(device)
        self.out_f32 = out_f32
        self.max_rows = max_rows or spec.max_rows
        self.desc = desc_of(spec, self.max_rows, out_f32)
        self.plan, self.ws_bytes = md.moe_decode_plan(self.desc)
        # Destroyed with the object, or at interpreter exit before the
        # binding module is torn down.
        self._release = weakref.finalize(self, md.lib().moe_decode_plan_destroy, self.plan)
        self.layout = md.moe_decode_workspace_layout(self.plan)
        base = {
            "router": to_device(layer.router, device), "bias": to_device(layer.expert_bias, device),
            "sh_gate": to_device(layer.sh_gate, device), "sh_up": to_device(layer.sh_up, device),
            "sh_down": to_device(layer.sh_down, device),
            "sh_gate_vec": to_device(layer.sh_gate_vec, device),
            "pre_norm_w": to_device(layer.pre_norm_w, device),
            "router_norm_w": to_device(layer.router_norm_w, device),
        }
        for name in ("gate", "up", "down"):
            proj = getattr(layer, name)
            base[name] = to_device(proj.data, device)
            base[name + "_s"] = to_device(proj.scale, device)
            base[name + "_b"] = to_device(proj.bias, device)
            base[name + "_s2"] = to_device(proj.scale2, device)
        self.copies = [_Copy(base, spec.num_experts, self.device)]
        for _ in range(copies - 1):
            cl = {k: (None if v is None else v.clone()) for k, v in base.items()}
            self.copies.append(_Copy(cl, spec.num_experts, self.device))
        self._plan_other = None      # the same layer with the other output format, made on demand
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        md.moe_decode_workspace_init(self.plan, self.workspace.data_ptr(), self.ws_bytes,
                                     torch.cuda.current_stream(self.device).cuda_stream)

    @property
    def weights(self) -> md.moe_decode_weights:
        return self.copies[0].weights

    def _plan(self, out_f32: Optional[bool]):
        """The plan for the requested output format: this layer's own, or a
        second plan of the same layer with MOE_OUT_F32 toggled (same workspace)."""
        if out_f32 is None or bool(out_f32) == self.out_f32:
            return self.plan
        if self._plan_other is None:
            plan, ws = md.moe_decode_plan(desc_of(self.spec, self.max_rows, bool(out_f32)))
            weakref.finalize(self, md.lib().moe_decode_plan_destroy, plan)
            assert ws == self.ws_bytes
            self._plan_other = plan
        return self._plan_other

    def new_out(self, m: int, out_f32: Optional[bool] = None) -> torch.Tensor:
        f32 = self.out_f32 if out_f32 is None else bool(out_f32)
        dt = torch.float32 if (f32 or self.spec.act_fmt == "f32") else torch.int16
        return torch.empty((m, self.spec.hidden), dtype=dt, device=self.device)

    def forward(self, x: torch.Tensor, m: Optional[int] = None, out: Optional[torch.Tensor] = None,
                idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                copy: int = 0, stream: Optional[int] = None, events=None,
                out_f32: Optional[bool] = None) -> torch.Tensor:
        m = x.shape[0] if m is None else m
        if out is None:
            out = self.new_out(m, out_f32)
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        args = (self._plan(out_f32), self.copies[copy].weights, x.data_ptr(), m, out.data_ptr(),
                None if idx is None else idx.data_ptr(), None if w is None else w.data_ptr(),
                self.workspace.data_ptr(), self.ws_bytes, st)
        if events is None:
            md.moe_decode_forward(*args)
        else:
            md.moe_decode_forward_timed(*args, events)
        return out

    def ws_view(self, field: str, dtype, count: int) -> torch.Tensor:
        """A view of one workspace array (moe_decode_ws_layout field)."""
        off = getattr(self.layout, field)
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.workspace[off:off + nbytes].view(dtype)


def out_to_numpy(spec: LayerSpec, out: torch.Tensor) -> np.ndarray:
    """Device output -> float64 numpy (bf16 bits decoded here for comparison only)."""
    o = out.cpu()
    if o.dtype == torch.int16:
        o = (o.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        return o.astype(np.float64)
    return o.numpy().astype(np.float64)
