"""The C ABI on the host (no GPU needed): the library loads, exports every
entry point the header declares, validates descriptions, lays out the
workspace, and rejects bad forward calls before anything is launched."""
import ctypes as C
import subprocess

import pytest

from mixture_experts_decode_amd import moe_decode as md
from mixture_experts_decode_amd import synth
from mixture_experts_decode_amd.device import desc_of


def test_library_exports_every_declared_entry_point():
    names = md.header_entry_points()
    assert len(names) >= 10
    lib = md.lib()
    for n in names:
        assert hasattr(lib, n), n
    syms = subprocess.run(["nm", "-D", "--defined-only", md.LIB_PATH], capture_output=True,
                          text=True, check=True).stdout
    exported = {line.split()[-1] for line in syms.splitlines() if " T " in line}
    assert set(names) <= exported
    assert "gfx950" in md.moe_decode_version()


def _desc(**kw):
    spec = synth.WORKLOADS["qwen3_30b_a3b_bf16"]
    d = desc_of(spec)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,status", [
    ("hidden", 0, md.MOE_EINVAL),
    ("hidden", 2044, md.MOE_EUNSUPPORTED),
    ("num_experts", 257, md.MOE_EUNSUPPORTED),
    ("top_k", 17, md.MOE_EUNSUPPORTED),
    ("top_k", 0, md.MOE_EINVAL),
    ("max_rows", 257, md.MOE_EUNSUPPORTED),
    ("max_rows", 0, md.MOE_EINVAL),
    ("act_fmt", md.MOE_AFF4_G64, md.MOE_EINVAL),
    ("expert_fmt", 7, md.MOE_EINVAL),
    ("expert_fmt", 6, md.MOE_EINVAL),
    ("routing", 4, md.MOE_EINVAL),
    ("flags", 1 << 10, md.MOE_EINVAL),
    ("flags", md.MOE_SHARED_GATED, md.MOE_EINVAL),
    ("inter", 100, md.MOE_EUNSUPPORTED),
    ("inter", 1 << 19, md.MOE_EUNSUPPORTED),       # 2048 x 524288 bf16 = 2 GiB: past 32-bit ranges
])
def test_plan_rejects(field, value, status):
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(**{field: value}))
    assert ei.value.status == status
    assert md.moe_decode_last_error()


def test_plan_rejects_fp8_shapes():
    # Scale blocks of 128 x 128: H and I multiples of 128; above 32 rows bf16
    # activations only (the matrix-core path).
    for kw in (dict(inter=768 + 64), dict(hidden=2048 + 32), dict(max_rows=33, act_fmt=md.MOE_F32)):
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_plan(_desc(expert_fmt=md.MOE_FP8_B128, **kw))
        assert ei.value.status == md.MOE_EUNSUPPORTED, kw
    for rows in (1, 32, 256):
        plan, ws = md.moe_decode_plan(_desc(expert_fmt=md.MOE_FP8_B128, max_rows=rows))
        assert ws > 0
        md.lib().moe_decode_plan_destroy(plan)


def test_plan_rejects_4bit_shapes():
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(expert_fmt=md.MOE_AFF4_G64, inter=96))
    assert ei.value.status == md.MOE_EUNSUPPORTED
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(expert_fmt=md.MOE_MXFP4_B32, hidden=2048 + 16))
    assert ei.value.status == md.MOE_EUNSUPPORTED
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(flags=md.MOE_SHARED, shared_inter=0))
    assert ei.value.status == md.MOE_EUNSUPPORTED


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_plan_and_layout_for_every_workload(name):
    _check_plan_and_layout(synth.WORKLOADS[name])


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "llama4_wbf_bf16"])
def test_plan_and_layout_grouped_rows(name):
    _check_plan_and_layout(synth.WORKLOADS[name].replace(rows=(256,)))


def test_grouped_rows_limits():
    for kw in (dict(act_fmt=md.MOE_F32, expert_fmt=md.MOE_F32), dict(expert_fmt=md.MOE_F32),
               dict(act_fmt=md.MOE_F32, expert_fmt=md.MOE_MXFP4_B32), dict(hidden=2048 + 16),
               dict(inter=768 + 8)):
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_plan(_desc(max_rows=64, **kw))
        assert ei.value.status == md.MOE_EUNSUPPORTED, kw
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(max_rows=257))
    assert ei.value.status == md.MOE_EUNSUPPORTED
    for fmt in (md.MOE_BF16, md.MOE_MXFP4_B32, md.MOE_NVFP4_B16, md.MOE_AFF4_G64, md.MOE_FP8_B128):
        plan, ws = md.moe_decode_plan(_desc(max_rows=256, expert_fmt=fmt))
        md.moe_decode_plan_destroy(plan)


def _shared_parts(spec):
    # About 2048 of Is per part, at most 16 parts.
    return max(1, min(spec.shared_inter // 2048, 16))


def test_shared_down_parts():
    assert _shared_parts(synth.WORKLOADS["llama4_wbf_bf16"]) == 4
    assert _shared_parts(synth.WORKLOADS["qwen35_35b_a3b_mxfp4"]) == 1
    spec = synth.WORKLOADS["qwen3_30b_a3b_bf16"].replace(shared=True, shared_inter=65536, hidden=256)
    assert _shared_parts(spec) == 16
    _check_plan_and_layout(spec)


def _check_plan_and_layout(spec):
    plan, ws = md.moe_decode_plan(desc_of(spec))
    try:
        L = md.moe_decode_workspace_layout(plan)
        assert L.total == ws
        te = spec.max_rows * spec.top_k
        fields = [(L.sync, 64), (L.logits, spec.max_rows * (spec.num_experts + 1) * 8),
                  (L.topk_idx, te * 4), (L.topk_w, te * 4), (L.row_gate, spec.max_rows * 4),
                  (L.sorted_pair, te * 4), (L.expert_offsets, (spec.num_experts + 1) * 4),
                  (L.pair_to_perm, te * 4), (L.active_experts, min(te, spec.num_experts) * 4),
                  (L.active_count, 4), (L.slot_info, min(te, spec.num_experts) * 128),
                  (L.act, te * spec.inter * 4),
                  (L.shared_act, spec.max_rows * (spec.shared_inter if spec.shared else 0) * 4),
                  (L.shared_y, _shared_parts(spec) * spec.max_rows * (spec.hidden if spec.shared else 0) * 4),
                  (L.routed_y, te * spec.hidden * 4 if spec.max_rows > 32 else 0),
                  (L.normed_x, spec.max_rows * spec.hidden * (4 if spec.act_fmt == "f32" else 2)
                   if spec.pre_expert_norm else 0)]
        spans = sorted((o, o + max(n, 1)) for o, n in fields)
        for (a0, a1), (b0, _) in zip(spans, spans[1:]):
            assert a1 <= b0, "workspace arrays overlap"
        assert all(o % 256 == 0 for o, _ in fields)
        assert spans[-1][1] <= ws
        want = ["route", "gate_up", "down_blend"]
        n = md.moe_decode_num_stages(plan)
        assert [md.moe_decode_stage_name(plan, i) for i in range(n)] == want
        assert md.moe_decode_stage_name(plan, n) == ""
    finally:
        md.moe_decode_plan_destroy(plan)


def _weights_stub():
    # Host addresses only: the calls below must fail validation before any
    # use of them.
    w = md.moe_decode_weights()
    for f, _ in md.moe_decode_weights._fields_:
        setattr(w, f, 4096)
    return w


@pytest.mark.parametrize("m", [0, -1, 9])
def test_forward_rejects_m_out_of_range(m):
    plan, ws = md.moe_decode_plan(desc_of(synth.WORKLOADS["qwen3_30b_a3b_bf16"]))
    try:
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_forward(plan, _weights_stub(), 4096, m, 4096, None, None, 4096 * 256,
                                  ws, 0)
        assert ei.value.status == md.MOE_EINVAL
    finally:
        md.moe_decode_plan_destroy(plan)


def test_forward_rejects_bad_pointers_and_workspace():
    plan, ws = md.moe_decode_plan(desc_of(synth.WORKLOADS["qwen35_35b_a3b_mxfp4"]))
    try:
        def call(**kw):
            a = dict(w=_weights_stub(), x=4096, m=1, out=4096, ws=4096 * 256, ws_bytes=ws)
            a.update(kw)
            with pytest.raises(md.MoeDecodeError) as ei:
                md.moe_decode_forward(plan, a["w"], a["x"], a["m"], a["out"], None, None, a["ws"],
                                      a["ws_bytes"], 0)
            return ei.value.status
        assert call(x=None) == md.MOE_EINVAL
        assert call(x=4097) == md.MOE_EINVAL          # misaligned
        assert call(out=None) == md.MOE_EINVAL
        assert call(ws=None) == md.MOE_EWORKSPACE
        assert call(ws=4096 * 256 + 16) == md.MOE_EWORKSPACE
        assert call(ws_bytes=ws - 1) == md.MOE_EWORKSPACE
        for field in ("router_w", "gate_w", "down_s", "sh_up_w", "sh_gate_vec"):
            w = _weights_stub()
            setattr(w, field, None)
            assert call(w=w) == md.MOE_EINVAL, field
        lib = md.lib()
        assert lib.moe_decode_forward(plan, None, 4096, 1, 4096, None, None, 4096 * 256, ws,
                                      None) == md.MOE_EINVAL
        assert lib.moe_decode_forward(None, C.byref(_weights_stub()), 4096, 1, 4096, None, None,
                                      4096 * 256, ws, None) == md.MOE_EINVAL
        # An event count no arrangement uses (a start and a stop event per stage).
        ev = (C.c_void_p * 7)(*([4096] * 7))
        assert lib.moe_decode_forward_timed(plan, C.byref(_weights_stub()), 4096, 1, 4096, None,
                                            None, 4096 * 256, ws, None, ev, 7) == md.MOE_EINVAL
    finally:
        md.moe_decode_plan_destroy(plan)


def test_sigmoid_bias_needs_expert_bias():
    plan, ws = md.moe_decode_plan(desc_of(synth.WORKLOADS["lfm2_8b_a1b_aff4"]))
    try:
        w = _weights_stub()
        w.expert_bias = None
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_forward(plan, w, 4096, 1, 4096, None, None, 4096 * 256, ws, 0)
        assert ei.value.status == md.MOE_EINVAL
        w = _weights_stub()
        w.up_b = None
        with pytest.raises(md.MoeDecodeError):
            md.moe_decode_forward(plan, w, 4096, 1, 4096, None, None, 4096 * 256, ws, 0)
    finally:
        md.moe_decode_plan_destroy(plan)


def test_nvfp4_needs_scales_and_second_level_scales():
    plan, ws = md.moe_decode_plan(desc_of(synth.WORKLOADS["qwen35_35b_a3b_nvfp4"]))
    try:
        for field in ("gate_s", "down_s", "gate_scale2", "up_scale2", "down_scale2"):
            w = _weights_stub()
            setattr(w, field, None)
            with pytest.raises(md.MoeDecodeError) as ei:
                md.moe_decode_forward(plan, w, 4096, 1, 4096, None, None, 4096 * 256, ws, 0)
            assert ei.value.status == md.MOE_EINVAL, field
    finally:
        md.moe_decode_plan_destroy(plan)
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(_desc(expert_fmt=md.MOE_NVFP4_B16, hidden=2048 + 16))
    assert ei.value.status == md.MOE_EUNSUPPORTED


def test_fp8_needs_scale_tables():
    plan, ws = md.moe_decode_plan(desc_of(synth.WORKLOADS["qwen35_35b_a3b_fp8"]))
    try:
        for field in ("gate_s", "up_s", "down_s"):
            w = _weights_stub()
            setattr(w, field, None)
            with pytest.raises(md.MoeDecodeError) as ei:
                md.moe_decode_forward(plan, w, 4096, 1, 4096, None, None, 4096 * 256, ws, 0)
            assert ei.value.status == md.MOE_EINVAL, field
    finally:
        md.moe_decode_plan_destroy(plan)


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "tiny_f32"])
def test_plan_and_layout_pre_expert_norm(name):
    _check_plan_and_layout(synth.WORKLOADS[name].replace(pre_expert_norm=True))


def test_pre_expert_norm_validation():
    for eps in (-1.0, float("nan"), float("inf")):
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_plan(_desc(flags=md.MOE_NORM_TOPK | md.MOE_PRE_EXPERT_NORM, norm_eps=eps))
        assert ei.value.status == md.MOE_EINVAL, eps
    plan, ws = md.moe_decode_plan(_desc(flags=md.MOE_NORM_TOPK | md.MOE_PRE_EXPERT_NORM, norm_eps=1e-6))
    try:
        w = _weights_stub()
        w.pre_norm_w = None
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_forward(plan, w, 4096, 1, 4096, None, None, 4096 * 256, ws, 0)
        assert ei.value.status == md.MOE_EINVAL
    finally:
        md.moe_decode_plan_destroy(plan)


def test_single_launch_arrangement_is_refused(monkeypatch):
    # The persistent single-launch arrangement is switched off: asking for it
    # fails at plan time instead of launching it.
    monkeypatch.setenv("MOE_DECODE_VARIANT", "fused")
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_plan(desc_of(synth.WORKLOADS["qwen3_30b_a3b_bf16"]))
    assert ei.value.status == md.MOE_EUNSUPPORTED


def test_measurement_utilities_reject_bad_arguments():
    """Validation runs before anything is launched (no GPU needed)."""
    for args in ((4096, 8192, 100), (4100, 8192, 4096), (4096, 8200, 4096), (None, 8192, 4096)):
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_bench_copy(args[0], args[1], args[2], None)
        assert ei.value.status == md.MOE_EINVAL
    for args in ((4096, 100, 8192), (4100, 4096, 8192), (4096, 4096, None)):
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_bench_read(args[0], args[1], args[2], None)
        assert ei.value.status == md.MOE_EINVAL


def test_noalloc_forward_rejects_a_plan_past_its_array():
    # 16 experts of 8192 x 8192, top-16, 256 rows: the activations alone need
    # 256 * 16 * 8192 * 4 bytes, far past the 32 MiB array; rejected before
    # any device call.
    d = _desc(hidden=8192, num_experts=16, top_k=16, inter=8192, max_rows=256)
    plan, ws = md.moe_decode_plan(d)
    try:
        assert ws > 32 << 20
        w = md.moe_decode_weights()
        with pytest.raises(md.MoeDecodeError) as ei:
            md.moe_decode_forward_noalloc(plan, w, 256, 1, 256, None, None, 0)
        assert ei.value.status == md.MOE_EWORKSPACE
        assert "32" in md.moe_decode_last_error() or "33554432" in md.moe_decode_last_error()
    finally:
        md.lib().moe_decode_plan_destroy(plan)
