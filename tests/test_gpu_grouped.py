"""GPU parity of the grouped path (33 <= m <= 256 rows: matrix-core expert
products) against the oracle, through the C ABI.

Same bar as the fused decode path: expert indices equal bit for bit, weights
to 1e-6 relative, outputs within tol * rms(oracle) (2e-2 with bf16 output,
1e-4 with f32 output); the sort arrays equal the oracle's sort; and a row's
result is bitwise the same for every m the path serves.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_decode_amd import synth
from mixture_experts_decode_amd.device import DeviceLayer
from tests.test_gpu_parity import TOL, TOL_OUT_F32, check, check_sort, run, say, small

pytestmark = pytest.mark.gpu


def grouped_rows(dl, layer, x, rows, what, out_f32=False):
    spec = layer.spec
    ref = oracle.forward(layer, x[:max(rows)])
    outs = {}
    for m in rows:
        say(f"[gpu] grouped {what} m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL_OUT_F32 if out_f32 else TOL["bf16"], f"{what} m={m}")
        check_sort(dl, m, idx)
        outs[m] = got
    mmax = max(m for m in rows if m > 32)
    for m in rows:
        if m > 32:
            assert np.array_equal(outs[m], outs[mmax][:m]), f"{what}: rows differ between m={m} and m={mmax}"
    return outs


_GV = [(routing, before) for routing in ("softmax", "sigmoid_bias", "sigmoid_logit")
       for before in (False, True)]
G_VARIANTS = [v + (("none", "plain", "gated")[i % 3],) for i, v in enumerate(_GV)]


@pytest.mark.parametrize("routing,before,shared", G_VARIANTS)
def test_grouped_small_variant(routing, before, shared):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=192, shared_inter=160, routing=routing,
                 weight_before_ffn=before, norm_topk=routing != "sigmoid_logit", routed_scaling_factor=1.25,
                 shared=shared != "none", shared_gated=shared == "gated", rows=(256,))
    seed = G_VARIANTS.index((routing, before, shared)) + 300
    layer = synth.make_layer(spec, seed=seed, threads=4)
    x = layer.x(0)
    what = f"{routing}/before={before}/shared={shared}"
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        grouped_rows(dl, layer, x, (33, 64, 200, 256, 8), what + f" f32out={out_f32}", out_f32)
        del dl
    torch.cuda.empty_cache()


# 4-bit and fp8 experts: the dequantising matrix-core loaders, short (four
# tiles per down wave) and long (I > 2048) down rows.
_QV = [("mxfp4", "softmax", False, "gated", 192), ("mxfp4", "sigmoid_bias", True, "none", 4096),
       ("nvfp4", "sigmoid_logit", False, "plain", 192), ("nvfp4", "softmax", True, "gated", 4096),
       ("nvfp4", "sigmoid_bias", False, "none", 2048 + 32),
       ("aff4", "sigmoid_bias", False, "gated", 192), ("aff4", "softmax", True, "none", 4096),
       ("fp8", "softmax", False, "gated", 256), ("fp8", "sigmoid_bias", True, "none", 4096),
       ("fp8", "sigmoid_logit", False, "plain", 2048 + 128)]


@pytest.mark.parametrize("fmt,routing,before,shared,inter", _QV)
def test_grouped_4bit(fmt, routing, before, shared, inter):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=inter, shared_inter=160, expert_fmt=fmt,
                 routing=routing, weight_before_ffn=before, norm_topk=routing != "sigmoid_logit",
                 shared=shared != "none", shared_gated=shared == "gated", rows=(128,))
    layer = synth.make_layer(spec, seed=_QV.index((fmt, routing, before, shared, inter)) + 400, threads=4)
    x = layer.x(0)
    what = f"{fmt}/{routing}/before={before}/shared={shared}/I={inter}"
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        grouped_rows(dl, layer, x, (33, 128, 70), what + f" f32out={out_f32}", out_f32)
        del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "nvfp4"])
def test_grouped_geglu(fmt):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=192, shared_inter=160, expert_fmt=fmt,
                 activation="gelu", shared=True, shared_gated=True, rows=(96,))
    layer = synth.make_layer(spec, seed=600 + len(fmt), threads=4)
    x = layer.x(0)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        grouped_rows(dl, layer, x, (33, 96), f"geglu {fmt} f32out={out_f32}", out_f32)
        del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_grouped_pre_expert_norm(fmt):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=192, shared_inter=160, expert_fmt=fmt,
                 pre_expert_norm=True, shared=True, shared_gated=True, rows=(80,))
    layer = synth.make_layer(spec, seed=650 + len(fmt), threads=4)
    x = layer.x(0)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        grouped_rows(dl, layer, x, (33, 80), f"pre-norm {fmt} f32out={out_f32}", out_f32)
        del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,routing,bias", [("bf16", "sqrtsoftplus", True), ("mxfp4", "sqrtsoftplus", False),
                                            ("aff4", "softmax", None)])
def test_grouped_router_pre_norm_and_sqrtsoftplus(fmt, routing, bias):
    spec = small(hidden=256, num_experts=12, top_k=3, inter=192, shared_inter=160, expert_fmt=fmt,
                 routing=routing, route_bias=bias, router_pre_norm=True, shared=True, shared_gated=True,
                 rows=(80,))
    layer = synth.make_layer(spec, seed=670 + len(fmt) + len(routing), threads=4)
    x = layer.x(0)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        grouped_rows(dl, layer, x, (33, 80, 8), f"router pre-norm {fmt}/{routing} f32out={out_f32}", out_f32)
        del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("E,k,inter,hidden", [(256, 16, 64, 128), (2, 1, 96, 160), (4, 4, 128, 64),
                                              (1, 1, 64, 96)])
def test_grouped_pair_extremes(E, k, inter, hidden):
    # 4096 pairs over every expert; one or two experts holding all rows (the
    # longest runs of passes); k = E (every row on every expert).
    spec = small(hidden=hidden, num_experts=E, top_k=k, inter=inter, shared=True, shared_gated=True,
                 shared_inter=96, rows=(256,), w_std=0.1)
    layer = synth.make_layer(spec, seed=E * 100 + k)
    x = layer.x(0)
    dl = DeviceLayer(layer)
    grouped_rows(dl, layer, x, (256, 97, 33), f"E={E} k={k}")
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,rows", [("qwen3_30b_a3b_bf16", (256, 128, 64, 33)),
                                       ("llama4_wbf_bf16", (64, 48)),
                                       ("qwen35_35b_a3b_mxfp4", (40, 33)),
                                       ("qwen35_35b_a3b_nvfp4", (40, 33)),
                                       ("qwen35_35b_a3b_fp8", (64, 33)),
                                       ("lfm2_8b_a1b_aff4", (64, 33))])
def test_grouped_workload(name, rows):
    spec = synth.WORKLOADS[name].replace(rows=(max(rows),))
    say(f"[gpu] grouped workload {name}: generating")
    layer = synth.make_layer(spec, seed=2)
    x = layer.x(1)
    dl = DeviceLayer(layer)
    grouped_rows(dl, layer, x, rows, name)
    dl32 = DeviceLayer(layer, out_f32=True)
    grouped_rows(dl32, layer, x, (max(rows),), name + " f32out", out_f32=True)
    del dl, dl32
    torch.cuda.empty_cache()


def test_paths_agree_at_the_boundary():
    # m = 32 (fused decode path) and m = 33 (grouped path): the first 32 rows
    # agree within the tolerance (different accumulation orders), with equal
    # selections.
    spec = small(hidden=512, num_experts=16, top_k=4, inter=256, shared=True, shared_gated=True,
                 shared_inter=192, rows=(64,))
    layer = synth.make_layer(spec, seed=77)
    x = layer.x(0)
    ref = oracle.forward(layer, x[:33])
    dl = DeviceLayer(layer, out_f32=True)
    o32, i32, w32 = run(dl, x, 32)
    o33, i33, w33 = run(dl, x, 33)
    check(spec, o32, i32, w32, ref, 32, TOL_OUT_F32, "m=32")
    check(spec, o33, i33, w33, ref, 33, TOL_OUT_F32, "m=33")
    assert np.array_equal(i32, i33[:32]) and np.array_equal(w32, w33[:32])
    r = np.abs(ref.out[:32])
    assert np.max(np.abs(o32 - o33[:32])) <= 2 * TOL_OUT_F32 * float(np.sqrt(np.mean(r * r)))
