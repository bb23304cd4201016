"""GPU parity: the HIP path (through the C ABI) against the oracle.

Expert indices must equal the oracle's bit for bit (slot order included),
routing weights agree to 1e-6 relative, and outputs satisfy
max|gpu - oracle| <= tol * rms(oracle) with tol = 2e-2 for bf16 activations
and 1e-5 for the fp32 path.  Sizes: every workload at every row count it
lists, plus small ragged layers over every format / routing / placement /
shared-expert variant and every kernel variant the host can pick.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_decode_amd import moe_decode as md
from mixture_experts_decode_amd import synth
from mixture_experts_decode_amd.device import DeviceLayer, out_to_numpy, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
# With MOE_OUT_F32 the bf16-activation path is only limited by fp32
# accumulation (inputs and dequantised weights are exact): a tighter bound.
TOL_OUT_F32 = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


SYNC_WORDS = 512                 # reserved completion words of the workspace


def check_sync_words(dl):
    """The reserved completion words are zero after a call, but word 2: the
    tag of the call whose routing was published (odd), or zero before any."""
    words = dl.ws_view("sync", torch.int32, SYNC_WORDS).cpu().numpy()
    assert words[2] == 0 or words[2] & 1, f"published tag {words[2]:#x} is not a tag"
    rest = np.delete(words, 2)
    assert not rest.any(), f"completion words not zero: {np.nonzero(words)[0][:8]}"


class Out(np.ndarray):
    """A forward's output as float64.  For a bf16 output, ``out32`` holds the
    float32 output of the same call on the same layer's MOE_OUT_F32 plan."""
    out32 = None


def run(dl: DeviceLayer, x_np: np.ndarray, m: int):
    """One forward of the first m rows.  A bf16 output is also checked, bit
    for bit, to be the round-to-nearest-even bf16 of the float32 output the
    same inputs give on the layer's MOE_OUT_F32 plan: the kernels compute one
    float32 value and only its store differs."""
    spec = dl.spec
    x = to_device(np.ascontiguousarray(x_np[:m]), "cuda")
    out = dl.new_out(m)
    idx = torch.full((m, spec.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((m, spec.top_k), float("nan"), dtype=torch.float32, device="cuda")
    dl.forward(x, m, out, idx, w)
    torch.cuda.synchronize()
    check_sync_words(dl)
    got = out_to_numpy(spec, out).view(Out)
    if spec.act_fmt == "bf16" and not dl.out_f32:
        o32 = dl.new_out(m, out_f32=True)
        dl.forward(x, m, o32, out_f32=True)
        torch.cuda.synchronize()
        check_sync_words(dl)
        o32 = o32.cpu()
        want = o32.to(torch.bfloat16).view(torch.int16).numpy()
        have = out.cpu().numpy()
        bad = np.nonzero(have != want)
        assert bad[0].size == 0, (f"bf16 output is not the bf16 rounding of the float32 output at "
                                  f"{bad[0][0], bad[1][0]}: {have[bad][0]:#06x} vs {want[bad][0]:#06x}")
        got.out32 = o32.numpy().astype(np.float64)
    return got, idx.cpu().numpy(), w.cpu().numpy()


# A bf16 output cannot be nearer the oracle's exact value than its own
# rounding, half a bf16 unit in the last place: up to 2^-8 |ref|, which
# exceeds 2e-2 rms(ref) once |ref| passes about 5 rms.  The 2e-2 bound is
# therefore checked on every element with |ref| <= BF16_STRICT_RMS * rms(ref),
# where that rounding (below 1.6e-2 rms) fits inside it; every element,
# outliers included, is covered by the two exact statements of ``run`` and
# ``check``: the bf16 output is the correctly rounded float32 output, and the
# float32 output is within TOL_OUT_F32 * rms(ref) of the oracle.
BF16_STRICT_RMS = 4.0


def check(spec, got, idx, w, ref, m, tol, what=""):
    """Indices exact, weights to 1e-6, and |gpu - oracle| <= tol * rms(oracle)
    elementwise.  When ``got`` carries the same call's float32 output (a bf16
    output, see ``run``), that output must be within TOL_OUT_F32 * rms
    everywhere, and the bf16 output within tol * rms wherever
    |ref| <= BF16_STRICT_RMS * rms."""
    assert np.array_equal(idx, ref.idx[:m]), f"{what}: expert indices differ\n{idx}\n{ref.idx[:m]}"
    werr = np.abs(w.astype(np.float64) - ref.w[:m])
    assert np.all(werr <= 1e-6 * np.abs(ref.w[:m]) + 1e-12), f"{what}: weights {werr.max()}"
    r = ref.out[:m]
    out32 = getattr(got, "out32", None)
    strict = np.ones(r.shape, bool) if out32 is None else np.abs(r) <= BF16_STRICT_RMS * rms(r)
    for val, t, name, where in ((np.asarray(got), tol, "out", strict),
                                (out32, TOL_OUT_F32, "f32 out", np.ones(r.shape, bool))):
        if val is None:
            continue
        diff = np.where(where, np.abs(val - r), 0.0)
        bound = t * rms(r)
        worst = int(np.argmax(diff))
        assert diff.flat[worst] <= bound, (f"{what} ({name}): |diff| {diff.flat[worst]:.3e} > {bound:.3e}"
                                           f" at {np.unravel_index(worst, diff.shape)} (|ref| {abs(r.flat[worst]):.3e},"
                                           f" rms {rms(r):.3e})")
    return float(np.abs(np.asarray(got) - r).max()) / max(rms(r), 1e-300)


def check_sort(dl, m, idx, records=True):
    """The workspace's sort arrays against the oracle's sort of the same
    selection; with records, also the slot records (fused decode path)."""
    spec = dl.spec
    te = m * spec.top_k
    want = oracle.sort_pairs(idx, spec.num_experts)
    sp = dl.ws_view("sorted_pair", torch.int32, te).cpu().numpy()
    off = dl.ws_view("expert_offsets", torch.int32, spec.num_experts + 1).cpu().numpy()
    p2p = dl.ws_view("pair_to_perm", torch.int32, te).cpu().numpy()
    cnt = int(dl.ws_view("active_count", torch.int32, 1).cpu().numpy()[0])
    act = dl.ws_view("active_experts", torch.int32, max(cnt, 1)).cpu().numpy()[:cnt]
    assert np.array_equal(sp, want["sorted_pair"])
    assert np.array_equal(off, want["expert_offsets"])
    assert np.array_equal(p2p, want["pair_to_perm"])
    assert cnt == want["active_count"] and np.array_equal(act, want["active_experts"])
    if not records:
        return
    # One 128-byte record per active slot: expert, pair range, the call's
    # tag (odd), the expert's table entries, then zero padding.
    recs = dl.ws_view("slot_info", torch.int32, max(cnt, 1) * 32).cpu().numpy().reshape(-1, 32)[:cnt]
    ptrs = recs.view(np.int64)
    tabs = {k: v.cpu().numpy() for k, v in dl.copies[0].tables.items()}
    names = ("gate", "up", "gate_s", "up_s", "gate_b", "up_b", "down", "down_s", "down_b")
    for u, e in enumerate(act):
        n_e = off[e + 1] - off[e]
        assert list(recs[u, :3]) == [e, off[e], n_e] and recs[u, 3] & 1, f"slot {u}: {recs[u, :4]}"
        assert recs[u, 3] == recs[0, 3], "one tag per call"
        for f, name in enumerate(names):
            assert ptrs[u, 2 + f] == (tabs[name][e] if name in tabs else 0), f"slot {u}: {name}"
        assert not recs[u, 22:].any()


# --------------------------------------------------------------- workloads

@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity_all_rows(name):
    spec = synth.WORKLOADS[name]
    say(f"[gpu] workload {name}: generating")
    layer = synth.make_layer(spec, seed=0)
    x = layer.x(0)
    ref = oracle.forward(layer, x)       # rows are independent: one call serves every m
    say(f"[gpu] workload {name}: oracle done, min margin {ref.margin.min():.3e}")
    dl = DeviceLayer(layer)
    outs = {}
    for m in spec.rows:
        say(f"[gpu] workload {name} m={m}: forward")
        got, idx, w = run(dl, x, m)
        rel = check(spec, got, idx, w, ref, m, TOL[spec.act_fmt], f"{name} m={m}")
        check_sort(dl, m, idx)
        outs[m] = got
        say(f"[gpu] workload {name} m={m}: ok, max|diff|/rms = {rel:.2e}")
    # A row's result does not depend on m (bitwise, same kernels).
    mmax = max(spec.rows)
    for m in spec.rows:
        assert np.array_equal(outs[m], outs[mmax][:m]), f"{name}: rows differ between m={m} and m={mmax}"
    # Deterministic across calls.
    again, _, _ = run(dl, x, mmax)
    assert np.array_equal(again, outs[mmax])
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["qwen3_30b_a3b_bf16", "qwen35_35b_a3b_mxfp4", "qwen35_35b_a3b_nvfp4",
                                  "qwen35_35b_a3b_fp8", "lfm2_8b_a1b_aff4",
                                  "llama4_wbf_bf16"])
def test_workload_fp32_output_tight(name):
    spec = synth.WORKLOADS[name]
    layer = synth.make_layer(spec, seed=1)
    x = layer.x(3)
    m = min(8, spec.max_rows)
    ref = oracle.forward(layer, x[:m])
    say(f"[gpu] workload {name} (f32 out) m={m}: forward")
    dl = DeviceLayer(layer, out_f32=True)
    got, idx, w = run(dl, x, m)
    rel = check(spec, got, idx, w, ref, m, TOL_OUT_F32, f"{name} f32-out")
    say(f"[gpu] workload {name} f32-out: max|diff|/rms = {rel:.2e}")
    del dl
    torch.cuda.empty_cache()


# ------------------------------------------------------ small ragged layers

def small(**kw):
    base = dict(name="small", hidden=320, num_experts=12, top_k=3, inter=192, shared_inter=136,
                act_fmt="bf16", expert_fmt="bf16", routing="softmax", norm_topk=True,
                w_std=0.05, rows=(8,))
    base.update(kw)
    return synth.LayerSpec(**base)


# Every (activation, expert format, routing, placement) combination once; the
# shared-expert variant (none / ungated / gated) rotates through them.
_BASE = [(act, fmt, routing, before)
         for act in ("f32", "bf16") for fmt in ("f32", "bf16", "aff4", "mxfp4")
         for routing in ("softmax", "sigmoid_bias", "sigmoid_logit") for before in (False, True)]
_BASE += [(act, "nvfp4", routing, before)
          for act in ("f32", "bf16") for routing in ("softmax", "sigmoid_bias", "sigmoid_logit")
          for before in (False, True)]
# The sqrt-softplus router over every format, with and without an expert bias.
_BASE += [(act, fmt, "sqrtsoftplus", before)
          for act in ("f32", "bf16") for fmt in ("f32", "bf16", "aff4", "mxfp4", "nvfp4")
          for before in (False, True)]
VARIANTS = [b + (("none", "plain", "gated")[i % 3],) for i, b in enumerate(_BASE)]

# fp8 experts (H and I multiples of 128: 3 x 2 scale blocks per gate/up
# matrix, 2 x 3 per down) over every routing, with the expert activation,
# the pre-expert norm and the router pre-norm rotating through the cases.
_FP8 = [(act, routing, before) for act in ("f32", "bf16")
        for routing in ("softmax", "sigmoid_bias", "sigmoid_logit", "sqrtsoftplus") for before in (False, True)]


@pytest.mark.parametrize("act,routing,before", _FP8)
def test_small_fp8(act, routing, before):
    i = _FP8.index((act, routing, before))
    shared = ("none", "plain", "gated")[i % 3]
    spec = small(act_fmt=act, expert_fmt="fp8", hidden=384, inter=256, shared_inter=136, routing=routing,
                 weight_before_ffn=before, norm_topk=routing != "sigmoid_logit", routed_scaling_factor=1.25,
                 shared=shared != "none", shared_gated=shared == "gated",
                 route_bias=(i % 2 == 0) if routing == "sqrtsoftplus" else None,
                 activation="gelu" if i % 4 == 1 else "silu", pre_expert_norm=i % 5 == 2,
                 router_pre_norm=i % 5 == 3)
    layer = synth.make_layer(spec, seed=700 + i, threads=4)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    what = f"fp8 {act}/{routing}/before={before}/shared={shared}/{spec.activation}"
    say(f"[gpu] small {what}")
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        for m in (1, 5, 8):
            got, idx, w = run(dl, x, m)
            tol = TOL[act] if not out_f32 else (TOL_OUT_F32 if act == "bf16" else TOL["f32"])
            check(spec, got, idx, w, ref, m, tol, f"{what} m={m} f32out={out_f32}")
            check_sort(dl, m, idx)


@pytest.mark.parametrize("act,fmt,routing,before,shared", VARIANTS)
def test_small_variant(act, fmt, routing, before, shared):
    i = VARIANTS.index((act, fmt, routing, before, shared))
    spec = small(act_fmt=act, expert_fmt=fmt, routing=routing, weight_before_ffn=before,
                 norm_topk=routing != "sigmoid_logit", routed_scaling_factor=1.25,
                 shared=shared != "none", shared_gated=shared == "gated",
                 route_bias=(i % 2 == 0) if routing == "sqrtsoftplus" else None)
    seed = VARIANTS.index((act, fmt, routing, before, shared)) + 100
    layer = synth.make_layer(spec, seed=seed, threads=4)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    what = f"{act}/{fmt}/{routing}/before={before}/shared={shared}"
    say(f"[gpu] small {what}")
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        for m in (1, 5, 8):
            got, idx, w = run(dl, x, m)
            tol = TOL[act] if not out_f32 else (TOL_OUT_F32 if act == "bf16" else TOL["f32"])
            check(spec, got, idx, w, ref, m, tol, f"{what} m={m} f32out={out_f32}")
            check_sort(dl, m, idx)


@pytest.mark.parametrize("act,fmt,routing", [("bf16", "bf16", "softmax"), ("bf16", "mxfp4", "sigmoid_bias"),
                                            ("bf16", "nvfp4", "softmax"), ("bf16", "aff4", "sigmoid_logit"),
                                            ("f32", "f32", "softmax"), ("f32", "nvfp4", "sigmoid_bias")])
def test_small_geglu(act, fmt, routing):
    # GeGLU experts (routed and shared): the exact GELU against the oracle's.
    spec = small(act_fmt=act, expert_fmt=fmt, routing=routing, activation="gelu", shared=True,
                 shared_gated=True, norm_topk=routing != "sigmoid_logit")
    layer = synth.make_layer(spec, seed=500 + len(act) + len(fmt) + len(routing), threads=4)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        for m in (1, 5, 8):
            say(f"[gpu] geglu {act}/{fmt}/{routing} m={m} f32out={out_f32}")
            got, idx, w = run(dl, x, m)
            tol = TOL[act] if not out_f32 else (TOL_OUT_F32 if act == "bf16" else TOL["f32"])
            check(spec, got, idx, w, ref, m, tol, f"geglu {act}/{fmt} m={m}")


@pytest.mark.parametrize("act,fmt,routing,before", [("bf16", "bf16", "softmax", False),
                                                   ("bf16", "nvfp4", "sigmoid_bias", True),
                                                   ("bf16", "aff4", "softmax", False),
                                                   ("f32", "f32", "sigmoid_logit", True)])
def test_small_pre_expert_norm(act, fmt, routing, before):
    # The experts read the RMS-normed rows (written in the activation format),
    # the router and the shared gate the raw rows.
    spec = small(act_fmt=act, expert_fmt=fmt, routing=routing, weight_before_ffn=before,
                 pre_expert_norm=True, shared=True, shared_gated=True,
                 norm_topk=routing != "sigmoid_logit")
    layer = synth.make_layer(spec, seed=700 + len(fmt) + len(routing) + before, threads=4)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        for m in (1, 5, 8):
            say(f"[gpu] pre-norm {act}/{fmt}/{routing}/before={before} m={m} f32out={out_f32}")
            got, idx, w = run(dl, x, m)
            tol = TOL[act] if not out_f32 else (TOL_OUT_F32 if act == "bf16" else TOL["f32"])
            check(spec, got, idx, w, ref, m, tol, f"pre-norm {act}/{fmt} m={m}")


@pytest.mark.parametrize("act,fmt,routing,expert_norm,before", [
    ("bf16", "bf16", "softmax", False, False), ("bf16", "mxfp4", "sqrtsoftplus", True, True),
    ("bf16", "aff4", "sigmoid_bias", False, False), ("bf16", "nvfp4", "sigmoid_logit", True, True),
    ("f32", "f32", "sqrtsoftplus", False, False), ("f32", "bf16", "softmax", True, False)])
def test_small_router_pre_norm(act, fmt, routing, expert_norm, before):
    # The router reads the rows RMS-normed with its own weight; the experts
    # read them raw or through the pre-expert norm; the shared gate reads them raw.
    spec = small(act_fmt=act, expert_fmt=fmt, routing=routing, router_pre_norm=True,
                 pre_expert_norm=expert_norm, weight_before_ffn=before, shared=True, shared_gated=True,
                 norm_topk=routing != "sigmoid_logit", route_bias=True if routing == "sqrtsoftplus" else None)
    layer = synth.make_layer(spec, seed=800 + len(fmt) + len(routing) + 2 * expert_norm + before, threads=4)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    for out_f32 in (False, True):
        dl = DeviceLayer(layer, out_f32=out_f32)
        for m in (1, 5, 8):
            say(f"[gpu] router pre-norm {act}/{fmt}/{routing}/expert_norm={expert_norm} m={m} f32out={out_f32}")
            got, idx, w = run(dl, x, m)
            tol = TOL[act] if not out_f32 else (TOL_OUT_F32 if act == "bf16" else TOL["f32"])
            check(spec, got, idx, w, ref, m, tol, f"router pre-norm {act}/{fmt} m={m}")
            check_sort(dl, m, idx)


@pytest.mark.parametrize("E,k,m", [(8, 3, 1), (256, 8, 8)])
def test_zero_input_ties_sqrtsoftplus(E, k, m):
    # x = 0: every score sqrt(ln 2): experts 0..k-1; normalised weights 1/k.
    spec = small(num_experts=E, top_k=k, routing="sqrtsoftplus", norm_topk=True, rows=(m,))
    layer = synth.make_layer(spec, seed=18)
    x = np.zeros((m, 320), np.uint16)
    say(f"[gpu] sqrt-softplus ties E={E} k={k} m={m}")
    got, idx, w = run(DeviceLayer(layer), x, m)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (m, 1)))
    assert np.allclose(w, 1.0 / k, rtol=1e-6, atol=0) and np.all(got == 0.0)


def test_every_row_count_and_pass_variant():
    spec = small(hidden=256, num_experts=16, top_k=4, inter=128, shared=True, shared_gated=True,
                 shared_inter=96, rows=(32,))
    layer = synth.make_layer(spec, seed=7)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    full = None
    for m in range(32, 0, -1):
        say(f"[gpu] m sweep m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"m={m}")
        check_sort(dl, m, idx)
        if full is None:
            full = got
        assert np.array_equal(got, full[:m])


# The matrix-core shared expert at several H and Is: short and long Is (a
# long one splits the down over parts of Is; at m = 1 a wave's share of at
# least 256 goes through the LDS ring, 1056 with a partial last batch), one
# and two column tiles (m <= 16, m > 16).
@pytest.mark.parametrize("hidden,shared_inter", [(1024, 512), (512, 1024), (256, 96), (512, 4096),
                                                 (256, 1056)])
def test_shared_expert_shapes(hidden, shared_inter):
    spec = small(hidden=hidden, num_experts=8, top_k=2, inter=64, shared=True, shared_gated=True,
                 shared_inter=shared_inter, rows=(32,))
    layer = synth.make_layer(spec, seed=hidden + shared_inter)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    say(f"[gpu] shared H={hidden} Is={shared_inter} m=32")
    full, idx, w = run(dl, x, 32)
    check(spec, full, idx, w, ref, 32, TOL["bf16"], f"shared H={hidden} Is={shared_inter} m=32")
    for m in (1, 5, 16, 17):
        say(f"[gpu] shared H={hidden} Is={shared_inter} m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"shared H={hidden} Is={shared_inter} m={m}")
        assert np.array_equal(got, full[:m])
    del dl
    torch.cuda.empty_cache()


# Long rows (I >= 4096) also take the split of each down row into parts.
@pytest.mark.parametrize("fmt,inter", [("bf16", 64), ("bf16", 256), ("bf16", 768), ("bf16", 1024),
                                       ("mxfp4", 512), ("mxfp4", 1024), ("aff4", 1792),
                                       ("aff4", 128), ("f32", 32), ("bf16", 4096),
                                       ("aff4", 8192), ("mxfp4", 4096), ("nvfp4", 96),
                                       ("nvfp4", 512), ("nvfp4", 4096), ("fp8", 128), ("fp8", 512),
                                       ("fp8", 1024), ("fp8", 4096)])
def test_down_lane_grouping(fmt, inter):
    spec = small(expert_fmt=fmt, inter=inter, hidden=512, num_experts=8, top_k=2,
                 act_fmt="f32" if fmt == "f32" else "bf16")
    layer = synth.make_layer(spec, seed=inter)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    for m in (1, 8):
        say(f"[gpu] lanes {fmt} I={inter} m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL[spec.act_fmt], f"{fmt} I={inter} m={m}")


def test_down_parts_are_a_plan_constant():
    # I = 8192, k = 8: a plan for one row splits each down row into 4 parts
    # of K, a plan for 32 rows into 2 (their partials share one LDS array).
    # Each plan gives a row the same bits for every m it serves; the two
    # plans agree with the oracle, and with each other within the tolerance.
    spec = small(hidden=256, num_experts=16, top_k=8, inter=8192, rows=(32,), shared=True, shared_gated=True,
                 shared_inter=256)
    layer = synth.make_layer(spec, seed=91)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    outs = {}
    for max_rows in (1, 32):
        dl = DeviceLayer(layer, max_rows=max_rows, out_f32=True)
        for m in sorted({1, max_rows}):
            say(f"[gpu] down parts: plan for {max_rows} rows, m={m}")
            got, idx, w = run(dl, x, m)
            check(spec, got, idx, w, ref, m, TOL_OUT_F32, f"plan {max_rows} m={m}")
            outs[(max_rows, m)] = got
        del dl
    assert np.array_equal(outs[(32, 1)], outs[(32, 32)][:1])
    r = ref.out[:1]
    assert np.max(np.abs(outs[(1, 1)] - outs[(32, 1)])) <= 2 * TOL_OUT_F32 * float(np.sqrt(np.mean(r * r)))
    torch.cuda.empty_cache()


def test_largest_pair_count_and_dense_limit():
    # E = 256, k = 16, m = 32: te = 512 pairs, the most the sort handles.
    spec = small(hidden=128, num_experts=256, top_k=16, inter=64, rows=(32,), w_std=0.1)
    layer = synth.make_layer(spec, seed=11)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    got, idx, w = run(dl, x, 32)
    check(spec, got, idx, w, ref, 32, TOL["bf16"], "te=512")
    check_sort(dl, 32, idx)
    # k = E: every expert active, weights are the full softmax.
    spec2 = small(hidden=128, num_experts=8, top_k=8, inter=64, rows=(4,))
    layer2 = synth.make_layer(spec2, seed=12)
    x2 = layer2.x(0)
    ref2 = oracle.forward(layer2, x2)
    dl2 = DeviceLayer(layer2)
    got, idx, w = run(dl2, x2, 4)
    check(spec2, got, idx, w, ref2, 4, TOL["bf16"], "k=E")


# (E, k, m): the first takes the rank selection (m * E small), the second the
# round-by-round wave selection.
@pytest.mark.parametrize("E,k,m", [(8, 3, 2), (256, 8, 8)])
def test_zero_input_and_ties(E, k, m):
    spec = small(num_experts=E, top_k=k, routing="softmax", rows=(m,))
    layer = synth.make_layer(spec, seed=13)
    x = np.zeros((m, spec.hidden), np.uint16)
    dl = DeviceLayer(layer)
    say(f"[gpu] ties E={E} k={k} m={m}")
    got, idx, w = run(dl, x, m)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (m, 1)))
    assert np.all(w == np.float32(1.0 / k)) and np.all(got == 0.0)
    # Duplicate router rows: the lower index ranks first.
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    win = int(ref.idx[0, 0])
    if win != 0:
        layer.router[0] = layer.router[win]
        ref = oracle.forward(layer, x)
        dl = DeviceLayer(layer)
        got, idx, w = run(dl, x, m)
        assert list(idx[0][:2]) == [0, win]
        check(spec, got, idx, w, ref, m, TOL["bf16"], "tie")


# Top-1 of many experts: the one-wave selection takes the wave maximum of the
# lanes' best high key words.  Random rows in every routing mode, then a tie
# on the winner (a duplicated router row: the lower index wins, through the
# full-order threshold) and x = 0 (every key equal: expert 0).
@pytest.mark.parametrize("routing", ["softmax", "sigmoid_bias", "sigmoid_logit", "sqrtsoftplus"])
def test_top1_many_experts(routing):
    spec = small(num_experts=256, top_k=1, routing=routing, norm_topk=routing != "sigmoid_logit",
                 weight_before_ffn=routing == "sigmoid_logit", rows=(1, 3, 8))
    layer = synth.make_layer(spec, seed=23)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    for m in (1, 3, 8):
        say(f"[gpu] top-1 of 256 {routing} m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"top-1 {routing} m={m}")
    win = int(ref.idx[0, 0])
    if win != 0:
        layer.router[0] = layer.router[win]
        if layer.expert_bias is not None:
            layer.expert_bias[0] = layer.expert_bias[win]
        ref = oracle.forward(layer, x)
        assert ref.idx[0, 0] == 0
        dl = DeviceLayer(layer)
        for m in (1, 3):
            say(f"[gpu] top-1 duplicated winner {routing} m={m}")
            got, idx, w = run(dl, x, m)
            check(spec, got, idx, w, ref, m, TOL["bf16"], f"top-1 tie {routing} m={m}")
    z = np.zeros((2, spec.hidden), np.uint16)
    if layer.expert_bias is not None:
        layer.expert_bias[:] = np.float32(0.25)
    dl = DeviceLayer(layer)
    for m in (1, 2):
        say(f"[gpu] top-1 x=0 {routing} m={m}")
        got, idx, w = run(dl, z, m)
        assert np.array_equal(idx, np.zeros((m, 1), np.int32)), idx
        assert np.array_equal(idx, oracle.forward(layer, z).idx[:m])


# Ties in the two sigmoid modes, at x = 0 (every logit 0).  (E, k, m) as
# above, plus m = 1, where every gate/up workgroup selects.
@pytest.mark.parametrize("E,k,m", [(8, 3, 1), (8, 3, 2), (256, 8, 1), (256, 8, 8)])
def test_zero_input_ties_sigmoid_modes(E, k, m):
    x = np.zeros((m, 320), np.uint16)
    # sigmoid + bias with equal biases: every key is sigma(0) + b, a tie
    # everywhere, so experts 0..k-1 in order; the normalised weights are 1/k.
    spec = small(num_experts=E, top_k=k, routing="sigmoid_bias", norm_topk=True, rows=(m,))
    layer = synth.make_layer(spec, seed=16)
    layer.expert_bias[:] = np.float32(0.25)
    say(f"[gpu] sigmoid+bias ties E={E} k={k} m={m}")
    got, idx, w = run(DeviceLayer(layer), x, m)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (m, 1)))
    assert np.all(w == np.float32(1.0 / k)) and np.all(got == 0.0)
    # Biases with repeated values: the selection is the top k of the bias,
    # ties to the lower index (a stable sort of -bias), weights still 1/k.
    rng = np.random.default_rng(E + k)
    layer.expert_bias[:] = (np.round(rng.standard_normal(E) * 2) / 8).astype(np.float32)
    order = np.argsort(-layer.expert_bias.astype(np.float64), kind="stable")[:k].astype(np.int32)
    got, idx, w = run(DeviceLayer(layer), x, m)
    assert np.array_equal(idx, np.tile(order, (m, 1))), (idx[0], order)
    assert np.array_equal(idx, oracle.forward(layer, x).idx)
    assert np.all(w == np.float32(1.0 / k)) and np.all(got == 0.0)
    # Raw logits with a sigmoid weight on the input, no normalisation:
    # experts 0..k-1, each weight sigma(0) = 1/2 exactly, output 0.
    spec = small(num_experts=E, top_k=k, routing="sigmoid_logit", norm_topk=False,
                 weight_before_ffn=True, shared=True, rows=(m,))
    layer = synth.make_layer(spec, seed=17)
    say(f"[gpu] raw-logit ties E={E} k={k} m={m}")
    got, idx, w = run(DeviceLayer(layer), x, m)
    assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (m, 1)))
    assert np.all(w == np.float32(0.5)) and np.all(got == 0.0)


# E >= 32 k: the pass variants that assume few pairs per active expert run
# up to m = 32, with a gated shared expert on the matrix cores (Is a multiple
# of 32) and on the vector units (Is not).
@pytest.mark.parametrize("shared_inter", [96, 104])
def test_row_sweep_many_experts(shared_inter):
    spec = small(hidden=256, num_experts=256, top_k=8, inter=128, shared=True, shared_gated=True,
                 shared_inter=shared_inter, rows=(32,))
    layer = synth.make_layer(spec, seed=19 + shared_inter)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    full = None
    for m in range(32, 0, -1):
        say(f"[gpu] E=256 k=8 Is={shared_inter} m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"Is={shared_inter} m={m}")
        check_sort(dl, m, idx)
        if full is None:
            full = got
        assert np.array_equal(got, full[:m]), f"rows differ between m={m} and m=32"
    del dl
    torch.cuda.empty_cache()



def test_row_sweep_many_experts_no_shared():
    """256 experts, top-8, no shared expert, m from 32 down to 1: above 8 rows
    the route launch runs on 16-wave workgroups (the top-k of up to 16 rows
    at once), at most 8 rows on 8-wave ones; every row matches the oracle and
    is bitwise the same at every m."""
    spec = small(hidden=256, num_experts=256, top_k=8, inter=128, shared=False, rows=(32,))
    layer = synth.make_layer(spec, seed=23)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    full = None
    for m in range(32, 0, -1):
        say(f"[gpu] E=256 k=8 no shared m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"no shared m={m}")
        check_sort(dl, m, idx)
        if full is None:
            full = got
        assert np.array_equal(got, full[:m]), f"rows differ between m={m} and m=32"
    del dl
    torch.cuda.empty_cache()

# The 4-bit workloads with 256 experts, up to the decode path's 32 rows.
@pytest.mark.parametrize("name", ["qwen35_35b_a3b_mxfp4", "qwen35_35b_a3b_nvfp4", "qwen35_35b_a3b_fp8"])
def test_workload_rows_to_32(name):
    spec = synth.WORKLOADS[name].replace(rows=(1, 8, 16, 17, 32))
    layer = synth.make_layer(spec, seed=0)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    dl = DeviceLayer(layer)
    outs = {}
    for m in spec.rows:
        say(f"[gpu] workload {name} (32 rows) m={m}")
        got, idx, w = run(dl, x, m)
        check(spec, got, idx, w, ref, m, TOL["bf16"], f"{name} m={m}")
        check_sort(dl, m, idx)
        outs[m] = got
    for m in spec.rows:
        assert np.array_equal(outs[m], outs[32][:m]), f"{name}: rows differ between m={m} and m=32"
    del dl
    torch.cuda.empty_cache()


def test_errors_launch_nothing():
    spec = small()
    layer = synth.make_layer(spec, seed=14)
    dl = DeviceLayer(layer)
    x = to_device(layer.x(0), "cuda")
    out = torch.full((8, spec.hidden), 12345, dtype=torch.int16, device="cuda")
    before = out.clone()
    for m in (0, 9):
        with pytest.raises(md.MoeDecodeError) as ei:
            dl.forward(x, m, out)
        assert ei.value.status == md.MOE_EINVAL
    with pytest.raises(md.MoeDecodeError) as ei:
        md.moe_decode_forward(dl.plan, dl.weights, x.data_ptr(), 1, out.data_ptr(), None, None,
                              dl.workspace.data_ptr(), dl.ws_bytes - 256, 0)
    assert ei.value.status == md.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(out, before)


def test_graph_replay_matches_eager():
    spec = synth.WORKLOADS["qwen35_35b_a3b_mxfp4"]
    layer = synth.make_layer(spec, seed=2)
    dl = DeviceLayer(layer)
    x = to_device(layer.x(0), "cuda")
    m = 8
    eager = dl.new_out(m)
    dl.forward(x, m, eager)
    torch.cuda.synchronize()
    out = dl.new_out(m)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dl.forward(x, m, out, stream=s.cuda_stream)
    for i in range(4):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        check_sync_words(dl)
        dl.forward(x, m, dl.new_out(m))      # eager work between replays
        torch.cuda.synchronize()


def test_measurement_utilities():
    """The copy reference copies exactly; the read reference leaves its sink alone."""
    n = (3 << 20) + 4                               # bytes: several grid strides and a tail
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    say("bench_copy / bench_read", n)
    md.moe_decode_bench_copy(src.data_ptr(), dst.data_ptr(), n - 4, 0)
    md.moe_decode_bench_read(src.data_ptr(), n - 4, sink.data_ptr(), 0)
    torch.cuda.synchronize()
    assert torch.equal(dst[:-1], src[:-1]) and int(dst[-1]) == 0
    assert int(sink[0]) in (7, 0x9E3779B9 - 2**32)


@pytest.mark.parametrize("name,rows", [("qwen3_30b_a3b_bf16", (1,)), ("qwen35_35b_a3b_mxfp4", (1,)),
                                       ("lfm2_8b_a1b_aff4", (1,)), ("tiny_f32", (1,)),
                                       ("llama4_wbf_bf16", (1,))])
def test_routing_placements_agree(name, rows, monkeypatch):
    """For one row, the routing computed by every gate/up workgroup and the
    routing computed once by the last router workgroup (the placement of
    every m > 1) give bitwise the same forward."""
    spec = synth.WORKLOADS[name]
    layer = synth.make_layer(spec, seed=5)
    x = layer.x(0)
    ref = oracle.forward(layer, x)
    res = {}
    for mode in ("gate_up", "once"):
        if mode == "once":
            monkeypatch.setenv("MOE_DECODE_ROUTE", mode)
        else:
            monkeypatch.delenv("MOE_DECODE_ROUTE", raising=False)
        dl = DeviceLayer(layer)
        for m in rows:
            say(f"[gpu] routing placement {mode} {name} m={m}")
            got, idx, w = run(dl, x, m)
            order = dl.ws_view("sorted_pair", torch.int32, m * spec.top_k).cpu().numpy()
            res[(mode, m)] = (got, idx, w, order)
            check(spec, got, idx, w, ref, m, TOL[spec.act_fmt], f"{mode} m={m}")
            check_sort(dl, m, idx)
    for m in rows:
        for a, b in zip(res[("gate_up", m)], res[("once", m)]):
            assert np.array_equal(a, b), f"placements differ at m={m}"

