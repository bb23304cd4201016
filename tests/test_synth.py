"""The seeded input generator: bf16 rounding, quantizers, determinism (CPU)."""
import numpy as np
import torch

from mixture_experts_decode_amd import synth
from tests import dense_ref


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        # exact ties: low 16 bits 0x8000 with even and odd kept mantissa
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], np.uint32)
         .view(np.float32)),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38], np.float32),
    ])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(f), want)


def test_mxfp4_quantizer_ties_to_even_and_saturates():
    vals = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -0.75, 0.1, 0.3] +
                    [0.0] * 20, np.float32)[None, :]
    packed, scale = synth.quantize_mxfp4(vals)
    assert scale[0, 0] == 127                     # amax 7 -> floor(log2 7) = 2 -> 2^0
    codes = np.empty(32, np.uint8)
    codes[0::2], codes[1::2] = packed[0] & 15, packed[0] >> 4
    assert list(codes[:12]) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 8 | 2, 0, 1]


def test_aff4_quantizer_reconstructs_within_half_step():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    packed, s, b = synth.quantize_aff4(w)
    proj = synth.Projection("aff4", 8, 256, packed[None], s[None], b[None])
    rec = dense_ref.dense_weight(proj, 0)
    step = np.repeat(dense_ref.bf16_to_f64(s), 64, axis=1)
    assert np.all(np.abs(rec - w) <= 0.51 * step + 1e-3 * step + np.abs(w) * 2 ** -8)


def test_generation_is_deterministic_and_thread_independent():
    spec = synth.LayerSpec(name="t", hidden=128, num_experts=6, top_k=2, inter=64,
                           expert_fmt="mxfp4", shared=True, shared_inter=64, shared_gated=True)
    a = synth.make_layer(spec, seed=5, threads=1)
    b = synth.make_layer(spec, seed=5, threads=8)
    for name in ("gate", "up", "down"):
        assert np.array_equal(getattr(a, name).data, getattr(b, name).data)
        assert np.array_equal(getattr(a, name).scale, getattr(b, name).scale)
    assert np.array_equal(a.router, b.router) and np.array_equal(a.sh_down, b.sh_down)
    c = synth.make_layer(spec, seed=6, threads=1)
    assert not np.array_equal(a.gate.data, c.gate.data)


def test_x_rows_are_a_prefix():
    spec = synth.WORKLOADS["qwen3_30b_a3b_bf16"]
    x8 = synth.make_x(spec, 0, 0)
    x1 = synth.make_x(spec, 0, 0, rows=1)
    assert x8.shape == (8, 2048) and np.array_equal(x1[0], x8[0])
    assert not np.array_equal(synth.make_x(spec, 0, 1), x8)


def test_workloads_are_valid():
    for spec in synth.WORKLOADS.values():
        synth.check_spec(spec)
        assert spec.top_k <= spec.num_experts


def test_nvfp4_quantizer_scales_and_error():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 64)) * 0.02).astype(np.float32)
    w[2, 16:32] = 0.0                                   # an all-zero block
    packed, sc, s2 = synth.quantize_nvfp4(w)
    assert packed.shape == (8, 32) and sc.shape == (8, 4) and s2.dtype == np.float32
    assert s2 == np.float32(np.abs(w).max() / (6.0 * 448.0))
    assert sc.max() <= 0x7E and sc[2, 1] == 0          # E4M3 at most 448; zero block -> scale 0
    codes = np.empty((8, 64), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = packed & 15, packed >> 4
    assert not codes[2, 16:32].any()
    proj = synth.Projection("nvfp4", 8, 64, packed[None], sc[None], scale2=np.array([s2]))
    from tests import dense_ref
    deq = dense_ref.dense_weight(proj, 0)
    # Each element within half an E2M1 step of its block scale (plus the
    # block scale's own rounding): a loose bound of 25% of the block maximum.
    blk = np.abs(w.astype(np.float64)).reshape(8, 4, 16).max(axis=2)
    err = np.abs(deq - w).reshape(8, 4, 16).max(axis=2)
    assert np.all(err <= 0.25 * blk + 1e-12)
    assert np.abs(deq - w).mean() < 0.1 * np.abs(w).mean()


def test_fp8_quantizer_scales_and_error():
    # Blocks of 128 x 128 with ragged edges (200 x 300 -> 2 x 3 blocks); each
    # block's scale maps its largest magnitude to 448 (the E4M3 maximum); an
    # all-zero block keeps scale 1 and code 0; every element is within half
    # an E4M3 step (relative 2^-4 of the element, or the subnormal step).
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((200, 300)) * 0.02).astype(np.float32)
    w[128:, 256:] = 0.0
    codes, sc = synth.quantize_fp8(w)
    assert codes.shape == (200, 300) and sc.shape == (2, 3) and sc.dtype == np.float32
    for i in range(2):
        for j in range(3):
            blk = np.abs(w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]).max()
            assert sc[i, j] == (np.float32(blk / 448.0) if blk > 0 else np.float32(1.0))
    assert not codes[128:, 256:].any()
    assert not np.any((codes & 0x7F) == 0x7F)            # no NaN codes: saturation at 448
    proj = synth.Projection("fp8", 200, 300, codes[None], sc[None])
    from tests import dense_ref
    deq = dense_ref.dense_weight(proj, 0)
    s_full = np.kron(sc.astype(np.float64), np.ones((128, 128)))[:200, :300]
    step = np.maximum(np.abs(w) * 2.0 ** -4, s_full * 2.0 ** -10)   # half a step, normal / subnormal
    assert np.all(np.abs(deq - w) <= step * (1 + 1e-6))
    assert np.array_equal(np.signbit(deq[w != 0]), np.signbit(w[w != 0]))
